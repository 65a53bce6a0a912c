// Attention for large blocks of queries (prompt prefill: many queries per KV
// head, causal among positions; [N] "nanoVLM における技術的実装", the prefill /
// decode split) on gfx950 matrix cores, fp16/bf16 storage, no split over keys.
//
// A workgroup takes ROWS = 16 * NW consecutive query rows of one (cache row,
// KV head) unit; wave w owns the 16-row tile w. The keys the workgroup's rows
// see, [0, kend), are staged through LDS in blocks of 64: every thread loads
// its share of a block's K and V rows (16-byte loads) into one of two
// register sets and writes it into LDS two iterations later, so each key is
// fetched from memory once per workgroup instead of once per wave and its
// loads have two iterations of compute to land. K runs one block ahead of V:
// the score products of block b + 1 are issued between block b's row maxima
// and its exponentials. LDS rows are 16-byte chunks XOR-swizzled by the row
// index, so the 16 rows of one operand load spread over the banks.
//
// Per 64-key block and tile (two 32-key halves), as the shared matrix-core
// tile computes each 32-key step:
//   S^T = K Q^T on v_mfma_f32_16x16x32 (lane l: scores of row l%16 against
//   keys 4*(l/16)+i of each 16-key half), online softmax per row in the log2
//   domain, O^T += V^T P^T with P fed as a high and a low part in the
//   storage type and V^T read from LDS with the transpose read.
// Rotated queries are rotated in fp32 at their positions, scaled by
// scale * log2(e), and fed as a high and a low part; stored queries are exact
// in the storage type and their scores are scaled after the product. Only
// the blocks a row's causal limit cuts through are masked; a wave skips the
// blocks its tile's rows do not see.
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
constexpr int kPrefillWaves = 4;              // waves per workgroup (one 16-row tile each)
constexpr int kXcdCus = 32;                   // CUs per XCD (256 CUs in 8 XCDs)

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

// Softmax weights as a high and a low bf16 part by truncation: hi = the
// upper half of each fp32, lo = the upper half of (p - hi), which is exact
// in fp32. Each truncation drops less than 2^-7 of its value, so hi + lo is
// within 2^-14 of p (rounding both to nearest: 2^-16), at three full-rate
// VALU operations per weight instead of two conversions and an unpack.
__device__ __forceinline__ void split_trunc_bf16(const float *x, u32x4 &hi, u32x4 &lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t a = __builtin_bit_cast(uint32_t, x[2 * e]);
    const uint32_t b = __builtin_bit_cast(uint32_t, x[2 * e + 1]);
    hi[e] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // (a's upper half, b's upper half << 16)
    const float ra = x[2 * e] - __builtin_bit_cast(float, a & 0xffff0000u);
    const float rb = x[2 * e + 1] - __builtin_bit_cast(float, b & 0xffff0000u);
    lo[e] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, rb), __builtin_bit_cast(uint32_t, ra), 0x07060302u);
  }
}

template <int DT, int NW, bool ROPE, bool RAGGED>
__global__ __launch_bounds__(64 * NW) void prefill_kernel(AttnArgs a) {
  constexpr int D = kHeadDim;
  constexpr int ROWB = D * 2;
  constexpr int ROWS = kMfmaRows * NW;
  constexpr int NT = 64 * NW;
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
  // y walks the row blocks from the longest down. Within an XCD the k-th
  // workgroup goes to CU k % 32 while all fit at once (measured), so CU j
  // holds the workgroups k = j, j + 32, j + 64, ...: the order is reversed
  // in every second round of 32, which pairs long blocks with short ones on
  // a CU (per-CU key blocks at most 11 instead of 14 on the 512-query GQA
  // prefill). Any other placement still gets every (unit, row block) once.
  int ux = blockIdx.x, y = blockIdx.y;
  if (gridDim.x % 8 == 0) {
    const int per = gridDim.x / 8;  // units per XCD
    const int k = blockIdx.x / 8 + per * blockIdx.y;
    const int K = per * gridDim.y;
    const int r = k / kXcdCus, j = k % kXcdCus;
    const int len = min(kXcdCus, K - r * kXcdCus);
    const int idx = (r & 1) ? r * kXcdCus + (len - 1 - j) : k;
    ux = 8 * (idx % per) + blockIdx.x % 8;
    y = idx / per;
  }
  const int unit = ux;
  const int bkv = unit / a.Hkv, hk = unit % a.Hkv;
  const RowSpan sp = row_span<RAGGED>(a, bkv);
  // Row block of this workgroup. Under a causal mask a block's work grows
  // with its position in its sequence; when blocks tile the sequences (the
  // rows of a unit are G / N sequences of N queries), y walks the position
  // blocks from the last down, every sequence's at each position in turn;
  // otherwise y walks the blocks from the last.
  int rb = (int)gridDim.y - 1 - y;
  if (sp.causal_base >= 0 && a.N % ROWS == 0) {
    const int bph = a.N / ROWS, nseq = a.G / a.N;
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

  // ---- staging through registers: chunk idx = tid + i * NT of a block is
  // row idx / 8, chunk idx % 8. Register set r holds K of block j + 1 and V
  // of block j (K runs one block ahead of V: the scores of block b + 1 are
  // taken while block b's softmax runs).
  u32x4 rk[2][CPT], rv[2][CPT];
  auto chunk_off = [&](int blk, int i) {
    const int idx = tid + i * NT;
    const int key = min(blk * kBlockKeys + idx / kChunks, kcap);
    return (uint32_t)key * ROWB + (idx % kChunks) * 16;
  };
  auto gload = [&](auto set, int j) {
    constexpr int r = decltype(set)::value;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      rk[r][i] = load16(kc + chunk_off(j + 1, i));
      rv[r][i] = load16(vc + chunk_off(j, i));
    }
  };
  auto lstore = [&](auto set, int kslot, int vslot) {
    constexpr int r = decltype(set)::value;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + i * NT;
      const int slot = swz(idx / kChunks, idx % kChunks);
      s_k[kslot][slot] = rk[r][i];
      s_v[vslot][slot] = rv[r][i];
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;

  // ---- the wave's query rows: lane l holds row l % 16 of the tile, dims
  // [8gq, +8) and [32 + 8gq, +8) (a rotary pair (i, i + 32) sits in one lane)
  const int grow = wg_g0 + wave * kMfmaRows + c;
  const bool active = grow < a.G;
  RowId rid{0, 0, 0};
  u32x4 qraw[2] = {u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};
  int lim = 0;
  if (active) {
    rid = row_id(a, bkv, hk, grow);
    const char *qrow = static_cast<const char *>(a.q) + out_row(a, rid) * 2;
    qraw[0] = load16(qrow + gq * 16);
    qraw[1] = load16(qrow + 64 + gq * 16);
    lim = (sp.causal_base < 0) ? sp.L : sp.causal_base + rid.i + 1;
  }
  // K(0) through set 1's K registers, then K(1) and V(0) (set 0)
#pragma unroll
  for (int i = 0; i < CPT; ++i) rk[1][i] = load16(kc + chunk_off(0, i));
  gload(Set0{}, 0);

  // the rows' limits over the tile: below tmin every row sees every key,
  // from tmax on no row sees any
  const int tmax = __builtin_amdgcn_readfirstlane((int)groups_max<1>((float)lim));
  const int tmin = __builtin_amdgcn_readfirstlane(
      -(int)groups_max<1>(-(float)(active ? lim : INT_MAX / 2)));

  // ---- query operands (rotated queries: fp32 rotation at the row's
  // position, then scale * log2(e), then a high and a low part)
  u32x4 qhi[2], qlo[2];
  if constexpr (ROPE) {
    float qc[8], qs[8], x0[8], x1[8];
    rope_cos_sin_run<8>(sp.causal_base + rid.i, gq * 8, RopeStep{a.rope_ratio}, qc, qs);
    unpack16<DT>(qraw[0], x0);
    unpack16<DT>(qraw[1], x1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      rope_rotate(x0[e], x1[e], qc[e], qs[e]);
      x0[e] *= a.scale_log2;
      x1[e] *= a.scale_log2;
    }
    split_hi_lo<DT>(x0, qhi[0], qlo[0]);
    split_hi_lo<DT>(x1, qhi[1], qlo[1]);
  } else {
    qhi[0] = qraw[0];
    qhi[1] = qraw[1];
    qlo[0] = qlo[1] = u32x4{0, 0, 0, 0};
  }

  float m = -INFINITY, lsum = 0.f;
  f32x4 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Scores S^T of the block in ring slot buf: st[h][t][i] = q_row . k_(s0 +
  // 32h + 16t + 4gq + i). K operand, half h, tile t, dims chunk kk: key
  // 32h + 16t + c, 16 bytes at dims 8gq + 32kk.
  using KOperand = u32x4[2][2][2];
  auto load_k = [&](const u32x4 *kbuf, KOperand &ka) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) ka[h][t][kk] = kbuf[swz(32 * h + 16 * t + c, gq + 4 * kk)];
  };
  auto scores = [&](const KOperand &ka, f32x4 (&st)[2][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        st[h][t] = mfma<DT>(ka[h][t][0], qhi[0], f32x4{0.f, 0.f, 0.f, 0.f});
        st[h][t] = mfma<DT>(ka[h][t][1], qhi[1], st[h][t]);
        if constexpr (ROPE) {
          st[h][t] = mfma<DT>(ka[h][t][0], qlo[0], st[h][t]);
          st[h][t] = mfma<DT>(ka[h][t][1], qlo[1], st[h][t]);
        }
      }
  };

  // Online softmax over the block's scores st (keys [s0, s0 + 64)), then O^T
  // += V^T P^T with V^T from ring slot vbuf. Its two 32-key halves share one
  // softmax update per row (one dependency chain per 64 keys instead of two
  // per 32).
  // mid() runs between the row maxima and the exponentials: the next
  // block's score products go there, so they overlap this block's softmax.
  auto softmax_pv = [&](const f32x4 (&st)[2][2], int s0, const u32x4 *vbuf, auto &&mid) {
    float sc[16];
    float mt = -INFINITY;
    const float mul = ROPE ? 1.f : a.scale_log2;
    if (s0 + kBlockKeys <= tmin) {  // every row sees every key of the block
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
        sc[j] = (key < lim) ? (ROPE ? v : v * mul) : -INFINITY;
        mt = fmaxf(mt, sc[j]);
      }
    }
    mt = groups_max<16>(mt);  // a row's keys sit in lanes c, c+16, c+32, c+48
    // lazy reference m (see online_update)
    const bool move = mt > m + kLazySoftmax;
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float mn = move ? mt : m;
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] *= alpha;
      lsum *= alpha;
      m = mn;
    }
    mid();
    // m = -inf only while every score so far is -inf (masked), and then
    // sc - (-FLT_MAX) is -inf too: p = 0 with no select per key
    const float mref = fmaxf(m, -FLT_MAX);
    float p[16];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      p[j] = __builtin_amdgcn_exp2f(sc[j] - mref);
      ps += p[j];
    }
    lsum += ps;
    // V^T operand, half h, dims 16t .. 16t + 15 (row c: dim 16t + c) against
    // the lane's 8 keys 32h + {4gq + j, 16 + 4gq + j} (j < 4), from two LDS
    // transpose reads: in each group of 16 lanes (one gq), lanes 4j .. 4j + 3
    // read the 32 bytes of dims 16t .. 16t + 15 of key j of the four, and
    // lane c receives dim 16t + c of all four keys
    const int tr_k = c & 3, tr_j = c >> 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 va[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x2 w[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int rr = 32 * h + 16 * u + 4 * gq + tr_j;
          const char *at = reinterpret_cast<const char *>(&vbuf[swz(rr, 2 * t + (tr_k >> 1))]) + 8 * (tr_k & 1);
          w[u] = __builtin_bit_cast(u32x2, lds_read_tr16(at));
        }
        va[t] = u32x4{w[0][0], w[0][1], w[1][0], w[1][1]};
      }
      u32x4 phi, plo;
      if constexpr (DT == BF16) split_trunc_bf16(p + 8 * h, phi, plo);
      else split_hi_lo<DT>(p + 8 * h, phi, plo);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        o[t] = mfma<DT>(va[t], phi, o[t]);
        o[t] = mfma<DT>(va[t], plo, o[t]);
      }
    }
  };

  // ---- blocks. LDS slot parity: K(j) in s_k[j % 2], V(j) in s_v[j % 2].
  // At the top of iteration b, after the barrier, K(b + 1) and V(b) are in
  // LDS and the register set b % 2 holds K(b + 2) and V(b + 1); the waves
  // write those into the slots that iteration b does not read (K(b)'s and
  // V(b - 1)'s, left by every wave at the barrier), refill the set with
  // K(b + 4) and V(b + 3), take the scores of block b + 1 and then block
  // b's softmax and P V. Each register set is written into LDS two
  // iterations after its loads went out. Loads and stores past the last
  // block fetch clamped rows into slots nobody reads, so every iteration
  // issues the same memory operations and the compiler's count of loads in
  // flight stays exact.
#pragma unroll
  for (int i = 0; i < CPT; ++i) s_k[0][swz((tid + i * NT) / kChunks, (tid + i * NT) % kChunks)] = rk[1][i];
  lstore(Set0{}, 1, 0);
  // the two sets' loads go out in the loop's order (set 0's, then set 1's),
  // so the waits the compiler derives at the loop head are the loop's own
  gload(Set0{}, 1);
  __builtin_amdgcn_sched_barrier(0);
  gload(Set1{}, 2);
  __syncthreads();
  f32x4 st[2][2];
  if (tmax > 0) {
    KOperand ka;
    load_k(s_k[0], ka);
    scores(ka, st);
  }
  // iteration b with register set P = b % 2
  auto iteration = [&](auto parity, int b) {
    constexpr int P = decltype(parity)::value;
    __syncthreads();
    lstore(parity, P, 1 - P);
    gload(parity, b + 3);
    const int s0 = b * kBlockKeys;
    if (s0 < tmax) {  // uniform: some row of the tile sees these keys
      // the next block's scores (past the tile's last block they are taken
      // over a slot of stale rows and never used: no branch in the softmax)
      KOperand ka;
      load_k(s_k[1 - P], ka);
      f32x4 st_next[2][2];
      softmax_pv(st, s0, s_v[P], [&] { scores(ka, st_next); });
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t) st[h][t] = st_next[h][t];
    }
  };
  for (int b = 0; b < nblocks; b += 2) {
    iteration(Set0{}, b);
    iteration(Set1{}, b + 1);
  }

  // ---- lane l holds O[row c][16t + 4gq + i] = o[t][i]
  const float l = groups_sum<16>(lsum);  // the row's keys were spread over the 4 lane groups
  if (active) {
    const float inv = 1.f / l;
    float *orow = a.out + out_row(a, rid) + 4 * gq;
#pragma unroll
    for (int t = 0; t < 4; ++t) store_f32x4(orow + 16 * t, o[t] * inv);
  }
}

template <int DT, bool ROPE>
void launch_rope(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.lens) launch_kernel(prefill_kernel<DT, kPrefillWaves, ROPE, true>, grid, block, s, a);
  else launch_kernel(prefill_kernel<DT, kPrefillWaves, ROPE, false>, grid, block, s, a);
}

template <int DT>
void launch_dt(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.rope_base > 0.f) launch_rope<DT, true>(a, grid, block, s);
  else launch_rope<DT, false>(a, grid, block, s);
}

}  // namespace

int prefill_rows_per_block() { return kMfmaRows * kPrefillWaves; }

hipError_t launch_prefill(int dtype, const AttnArgs &a, hipStream_t s) {
  const int rows = prefill_rows_per_block();
  const dim3 grid(a.Bkv * a.Hkv, (a.G + rows - 1) / rows);
  const dim3 block(64 * kPrefillWaves);
  if (dtype == F16) launch_dt<F16>(a, grid, block, s);
  else launch_dt<BF16>(a, grid, block, s);
  return hipGetLastError();
}

}  // namespace kvd
