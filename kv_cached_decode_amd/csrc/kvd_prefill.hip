// Attention for large blocks of queries (prompt prefill: many queries per KV
// head, causal among positions; [N] "nanoVLM における技術的実装", the prefill /
// decode split) on gfx950 matrix cores, fp16/bf16 storage, no split over keys.
//
// A workgroup takes ROWS = 16 * NW * TPW consecutive query rows of one (cache
// row, KV head) unit: wave w owns the TPW 16-row tiles w*TPW .. w*TPW+TPW-1.
// The keys the workgroup's rows see, [0, kend), are staged through LDS in
// blocks of 64: every thread loads its share of the next block's K and V
// rows (16-byte loads) two blocks ahead, in two register sets used in turn,
// and writes a block into the free LDS buffer while the waves compute on the
// other, so each key is fetched from memory once per workgroup instead of
// once per wave and its loads have two blocks of compute to land. LDS rows are 16-byte chunks
// XOR-swizzled by the row index, so the 16 rows of one operand load spread
// over the banks.
//
// Per 64-key block and tile (two 32-key halves), as the shared matrix-core
// tile computes each 32-key step:
//   S^T = K Q^T on v_mfma_f32_16x16x32 (lane l: scores of row l%16 against
//   keys 4*(l/16)+i of each 16-key half), online softmax per row in the log2
//   domain, O^T += V^T P^T with P fed as a high and a low part in the
//   storage type and V^T read from LDS with the transpose read.
// The K and V operands of a step are read from LDS once per wave and serve
// all TPW tiles. Rotated queries are rotated in fp32 at their positions,
// scaled by scale * log2(e), and fed as a high and a low part; stored
// queries are exact in the storage type and their scores are scaled after
// the product. Only the steps a row's causal limit cuts through are masked;
// a wave skips the steps its tiles' rows do not see.
#include <float.h>

#include <type_traits>

#include "kvd_attn_common.hpp"
#include "kvd_device.hpp"
#include "kvd_internal.hpp"
#include "kvd_mfma.hpp"

namespace kvd {

namespace {

constexpr int kBlockKeys = 64;                // keys staged in LDS per block
constexpr int kChunks = kHeadDim * 2 / 16;    // 16-byte chunks per K or V row
// Workgroup shape, measured on the GQA prefill (B8, 9/3 heads, 512 causal
// queries): 4 waves of one 16-row tile, 15.6 us; 2 or 8 waves of one tile
// 16.6 / 16.8 us; two tiles per wave (4 or 2 waves) far slower.
constexpr int kPrefillWaves = 4;              // waves per workgroup
constexpr int kPrefillTiles = 1;              // 16-row tiles per wave

// LDS slot of chunk ch of staged row r.
__device__ __forceinline__ int swz(int r, int ch) { return r * kChunks + (ch ^ (r & 7)); }

// LDS transpose read of 16-bit elements (ds_read_b64_tr_b16, gfx950): in
// each group of 16 lanes, the 8 bytes that lanes 4j .. 4j + 3 address form
// row j (16 elements, lane 4j + k's element e at column 4k + e) of a 4 x 16
// block, and lane c receives column c: element c of rows 0, 1, 2, 3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_read_tr16(const void *p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(__attribute__((address_space(3))) const char *)p);
}

template <int DT, int NW, int TPW, bool ROPE, bool RAGGED>
__global__ __launch_bounds__(64 * NW) void prefill_kernel(AttnArgs a) {
  constexpr int D = kHeadDim;
  constexpr int ROWB = D * 2;
  constexpr int NT = 64 * NW;
  constexpr int ROWS = kMfmaRows * NW * TPW;
  constexpr int CPT = kBlockKeys * kChunks / NT;  // K (and V) chunks per thread per block
  static_assert(DT != F32, "matrix-core tiles take 16-bit storage");
  static_assert(CPT >= 1 && CPT * NT == kBlockKeys * kChunks, "the block splits evenly");
  __shared__ u32x4 s_k[2][kBlockKeys * kChunks];
  __shared__ u32x4 s_v[2][kBlockKeys * kChunks];

  hoist_args(a);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, gq = lane >> 4;
  // Workgroup w runs on XCD w % 8 (workgroups are dealt to the 8 XCDs in
  // turn), and the linear id is x + gridDim.x * y: with the unit in x, each
  // XCD holds whole units (their keys stay in its own L2) and an even share
  // of long and short row blocks. With the row block in x instead, the last
  // block of every 8 (the longest under a causal mask) landed on one XCD.
  // The longest blocks go out first (the waves dispatched first issue first).
  const int unit = blockIdx.x;
  const int bkv = unit / a.Hkv, hk = unit % a.Hkv;
  const RowSpan sp = row_span<RAGGED>(a, bkv);
  // Row block of this workgroup. Under a causal mask a block's work grows
  // with its position in its sequence; when blocks tile the sequences (the
  // rows of a unit are G / N sequences of N queries), y walks the position
  // blocks from the last down, every sequence's at each position in turn;
  // otherwise y walks the blocks from the last.
  int rb = (int)gridDim.y - 1 - (int)blockIdx.y;
  if (sp.causal_base >= 0 && a.N % ROWS == 0) {
    const int bph = a.N / ROWS, nseq = a.G / a.N;
    const int y = blockIdx.y;
    rb = (y % nseq) * bph + (bph - 1 - y / nseq);
  }
  const size_t head = (size_t)bkv * a.Hkv + hk;
  const char *kc = static_cast<const char *>(a.k) + head * a.S_max * ROWB;
  const char *vc = static_cast<const char *>(a.v) + head * a.S_max * ROWB;
  const int wg_g0 = rb * ROWS;

  // ---- the workgroup's keys: [0, kend), kend the largest limit among its
  // rows (rows are numbered q * N + i, query i at position causal_base + i)
  int kend = sp.L;
  if (sp.causal_base >= 0) {
    const int g_hi = min(wg_g0 + ROWS, a.G) - 1;
    const int qa = (int)fast_div((uint32_t)wg_g0, a.div_N);
    const int qb = (int)fast_div((uint32_t)g_hi, a.div_N);
    const int imax = (qa != qb) ? a.N - 1 : g_hi - qb * a.N;
    kend = min(sp.L, sp.causal_base + imax + 1);
  }
  kend = __builtin_amdgcn_readfirstlane(kend);
  const int kcap = sp.L - 1;  // staged rows past the cache's valid rows repeat its last one
  const int nblocks = (kend + kBlockKeys - 1) / kBlockKeys;

  // ---- staging: chunk idx = tid + i * NT of a block is row idx / 8, chunk
  // idx % 8; block j goes through register set j % 2 and LDS buffer j % 2
  u32x4 rk[2][CPT], rv[2][CPT];
  auto gload = [&](auto set, int b) {
    constexpr int r = decltype(set)::value;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + i * NT;
      const int key = min(b * kBlockKeys + idx / kChunks, kcap);
      const uint32_t off = (uint32_t)key * ROWB + (idx % kChunks) * 16;
      rk[r][i] = load16(kc + off);
      rv[r][i] = load16(vc + off);
    }
  };
  auto lstore = [&](auto set) {
    constexpr int r = decltype(set)::value;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + i * NT;
      const int slot = swz(idx / kChunks, idx % kChunks);
      s_k[r][slot] = rk[r][i];
      s_v[r][slot] = rv[r][i];
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;

  // ---- the wave's query rows: lane l holds row l % 16 of each tile, dims
  // [8gq, +8) and [32 + 8gq, +8) (a rotary pair (i, i + 32) sits in one lane)
  u32x4 qraw[TPW][2];
  int lim[TPW];
  RowId rid[TPW];
  bool active[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int grow = wg_g0 + (wave * TPW + tt) * kMfmaRows + c;
    active[tt] = grow < a.G;
    rid[tt] = RowId{0, 0, 0};
    qraw[tt][0] = qraw[tt][1] = u32x4{0, 0, 0, 0};
    lim[tt] = 0;
    if (active[tt]) {
      rid[tt] = row_id(a, bkv, hk, grow);
      const char *qrow = static_cast<const char *>(a.q) + out_row(a, rid[tt]) * 2;
      qraw[tt][0] = load16(qrow + gq * 16);
      qraw[tt][1] = load16(qrow + 64 + gq * 16);
      lim[tt] = (sp.causal_base < 0) ? sp.L : sp.causal_base + rid[tt].i + 1;
    }
  }
  gload(Set0{}, 0);
  gload(Set1{}, 1);

  // the rows' limits over each tile: below tmin every row sees every key,
  // from tmax on no row sees any
  int tmin[TPW], tmax[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    tmax[tt] = __builtin_amdgcn_readfirstlane((int)groups_max<1>((float)lim[tt]));
    tmin[tt] = __builtin_amdgcn_readfirstlane(
        -(int)groups_max<1>(-(float)(active[tt] ? lim[tt] : INT_MAX / 2)));
  }

  // ---- query operands (rotated queries: fp32 rotation at the row's
  // position, then scale * log2(e), then a high and a low part)
  u32x4 qhi[TPW][2], qlo[TPW][2];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    if constexpr (ROPE) {
      float qc[8], qs[8], x0[8], x1[8];
      rope_cos_sin_run<8>(sp.causal_base + rid[tt].i, gq * 8, RopeStep{a.rope_step, a.rope_ratio},
                          qc, qs);
      unpack16<DT>(qraw[tt][0], x0);
      unpack16<DT>(qraw[tt][1], x1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        rope_rotate(x0[e], x1[e], qc[e], qs[e]);
        x0[e] *= a.scale_log2;
        x1[e] *= a.scale_log2;
      }
      split_hi_lo<DT>(x0, qhi[tt][0], qlo[tt][0]);
      split_hi_lo<DT>(x1, qhi[tt][1], qlo[tt][1]);
    } else {
      qhi[tt][0] = qraw[tt][0];
      qhi[tt][1] = qraw[tt][1];
      qlo[tt][0] = qlo[tt][1] = u32x4{0, 0, 0, 0};
    }
  }

  float m[TPW], lsum[TPW];
  f32x4 o[TPW][4];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    m[tt] = -INFINITY;
    lsum[tt] = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[tt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One staged block [s0, s0 + 64) of LDS buffer buf: its two 32-key halves
  // h go through the matrix cores together and share one softmax update per
  // row (one dependency chain per 64 keys instead of two per 32).
  auto block_step = [&](int buf, int s0) {
    bool any = false;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) any |= s0 < tmax[tt];
    if (!any) return;  // uniform
    // K operand, half h, tile t, dims chunk kk: key 32h + 16t + c, 16 bytes
    // at dims 8gq + 32kk
    u32x4 ka[2][2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          ka[h][t][kk] = s_k[buf][swz(32 * h + 16 * t + c, gq + 4 * kk)];
    // V^T operand, half h, dims 16t .. 16t + 15 (row c: dim 16t + c) against
    // the lane's 8 keys 32h + {4gq + j, 16 + 4gq + j} (j < 4), from two LDS
    // transpose reads: in each group of 16 lanes (one gq), lanes 4j .. 4j + 3
    // read the 32 bytes of dims 16t .. 16t + 15 of key j of the four, and
    // lane c receives dim 16t + c of all four keys
    u32x4 va[2][4];
    const int tr_k = c & 3, tr_j = c >> 2;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x2 w[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int rr = 32 * h + 16 * u + 4 * gq + tr_j;
          const char *at = reinterpret_cast<const char *>(&s_v[buf][swz(rr, 2 * t + (tr_k >> 1))]) +
                           8 * (tr_k & 1);
          w[u] = __builtin_bit_cast(u32x2, lds_read_tr16(at));
        }
        va[h][t] = u32x4{w[0][0], w[0][1], w[1][0], w[1][1]};
      }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      if (s0 >= tmax[tt]) continue;  // uniform: no row of the tile sees these keys
      // scores S^T: st[h][t][i] = q_row . k_(s0 + 32h + 16t + 4gq + i)
      f32x4 st[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          st[h][t] = mfma<DT>(ka[h][t][0], qhi[tt][0], f32x4{0.f, 0.f, 0.f, 0.f});
          st[h][t] = mfma<DT>(ka[h][t][1], qhi[tt][1], st[h][t]);
          if constexpr (ROPE) {
            st[h][t] = mfma<DT>(ka[h][t][0], qlo[tt][0], st[h][t]);
            st[h][t] = mfma<DT>(ka[h][t][1], qlo[tt][1], st[h][t]);
          }
        }
      float sc[16];
      float mt = -INFINITY;
      const float mul = ROPE ? 1.f : a.scale_log2;
      if (s0 + kBlockKeys <= tmin[tt]) {  // every row sees every key of the block
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float v = st[j >> 3][(j >> 2) & 1][j & 3];
          sc[j] = ROPE ? v : v * mul;
          mt = fmaxf(mt, sc[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = s0 + 16 * (j >> 2) + 4 * gq + (j & 3);
          const float v = st[j >> 3][(j >> 2) & 1][j & 3];
          sc[j] = (key < lim[tt]) ? (ROPE ? v : v * mul) : -INFINITY;
          mt = fmaxf(mt, sc[j]);
        }
      }
      mt = groups_max<16>(mt);  // a row's keys sit in lanes c, c+16, c+32, c+48
      // lazy reference m (see online_update)
      const bool move = mt > m[tt] + kLazySoftmax;
      if (__builtin_amdgcn_ballot_w64(move)) {
        const float mn = move ? mt : m[tt];
        const float alpha = (m[tt] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[tt] - mn);
#pragma unroll
        for (int t = 0; t < 4; ++t) o[tt][t] *= alpha;
        lsum[tt] *= alpha;
        m[tt] = mn;
      }
      // m = -inf only while every score so far is -inf (masked), and then
      // sc - (-FLT_MAX) is -inf too: p = 0 with no select per key
      const float mref = fmaxf(m[tt], -FLT_MAX);
      float p[16];
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        p[j] = __builtin_amdgcn_exp2f(sc[j] - mref);
        ps += p[j];
      }
      lsum[tt] += ps;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 phi, plo;
        split_hi_lo<DT>(p + 8 * h, phi, plo);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          o[tt][t] = mfma<DT>(va[h][t], phi, o[tt][t]);
          o[tt][t] = mfma<DT>(va[h][t], plo, o[tt][t]);
        }
      }
    }
  };

  // ---- blocks: compute on one LDS buffer while the other is filled from
  // the register set loaded two blocks earlier; one barrier per block (a
  // buffer is written only after every wave has left the block that read it)
  // Every load, store and barrier below is unconditional (blocks past the
  // last one load clamped rows, are written into a buffer nobody reads and
  // have no step to run), so the compiler's count of loads in flight stays
  // exact across the loop and each write waits only for the set it writes.
  lstore(Set0{});
  gload(Set0{}, 2);
  __syncthreads();
  // block b (parity P): compute, then block b + 1 into the other buffer and
  // block b + 3 into the register set that held it
  auto block = [&](auto parity, int b) {
    constexpr int P = decltype(parity)::value;
    block_step(P, b * kBlockKeys);
    lstore(std::integral_constant<int, 1 - P>{});
    gload(std::integral_constant<int, 1 - P>{}, b + 3);
    __syncthreads();
  };
  for (int b = 0; b < nblocks; b += 2) {
    block(Set0{}, b);
    block(Set1{}, b + 1);
  }

  // ---- lane l holds O[row c][16t + 4gq + i] = o[t][i]
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const float l = groups_sum<16>(lsum[tt]);  // the row's keys were spread over the 4 lane groups
    if (active[tt]) {
      const float inv = 1.f / l;
      float *orow = a.out + out_row(a, rid[tt]) + 4 * gq;
#pragma unroll
      for (int t = 0; t < 4; ++t) *reinterpret_cast<f32x4 *>(orow + 16 * t) = o[tt][t] * inv;
    }
  }
}

template <int DT, bool ROPE>
void launch_rope(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.lens) launch_kernel(prefill_kernel<DT, kPrefillWaves, kPrefillTiles, ROPE, true>, grid, block, s, a);
  else launch_kernel(prefill_kernel<DT, kPrefillWaves, kPrefillTiles, ROPE, false>, grid, block, s, a);
}

template <int DT>
void launch_dt(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.rope_base > 0.f) launch_rope<DT, true>(a, grid, block, s);
  else launch_rope<DT, false>(a, grid, block, s);
}

}  // namespace

int prefill_rows_per_block() { return kMfmaRows * kPrefillWaves * kPrefillTiles; }

hipError_t launch_prefill(int dtype, const AttnArgs &a, hipStream_t s) {
  const int rows = prefill_rows_per_block();
  const dim3 grid(a.Bkv * a.Hkv, (a.G + rows - 1) / rows);
  const dim3 block(64 * kPrefillWaves);
  if (dtype == F16) launch_dt<F16>(a, grid, block, s);
  else launch_dt<BF16>(a, grid, block, s);
  return hipGetLastError();
}

}  // namespace kvd
