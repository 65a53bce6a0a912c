// Decode attention for blocks of queries (N > 1: speculative verification,
// prompt prefill) on gfx950 matrix cores, fp16/bf16 storage.
//
// Both products run on v_mfma_f32_16x16x32 in their transposed form, so every
// lane works for a single query row:
//   S^T = K Q^T    A = 16 keys x 32 dims (a lane: one key, 8 contiguous dims
//                  = one 16-byte load), B = 32 dims x 16 query rows (a lane:
//                  one row, 8 dims); lane l ends with the scores of row l%16
//                  against keys 4*(l/16)+i of each 16-key tile.
//   O^T = V^T P^T  B = P^T: exactly the 8 probabilities lane l already holds
//                  (keys 4*(l/16)+i of the two 16-key tiles, taken in that
//                  order as the contraction index); A = V^T for 16 output dims,
//                  with the dims interleaved (dim 4c + t in row c of tile t)
//                  so that lane l reads the 8 bytes [4c, 4c+4) of each of its
//                  8 keys: 16 lanes cover a whole 128-byte V row. Lane l ends
//                  with O[row l%16][16*(l/16) .. +16).
// Softmax runs online per row in the log2 domain. P (and rotated queries) are
// fed to the MFMA as a high and a low part in the storage type, so their
// rounding stays far below the output tolerance; K, V and stored queries are
// exact in the storage type already.
//
// A workgroup of NW waves covers RW 16-row tiles: RW = NW = 4 (prefill: each
// wave its own rows, all keys of the chunk) or RW = 1 (verification: the 4 or
// 8 waves share the rows and take every NW-th 32-key step, merged in LDS).
// Splits over keys are merged as in the streaming kernel.
#include <stdlib.h>

#include "kvd_attn_common.hpp"
#include "kvd_device.hpp"
#include "kvd_internal.hpp"
#include "kvd_mfma.hpp"

namespace kvd {

namespace {

constexpr int kRows = kMfmaRows;  // query rows per MFMA tile
constexpr int kStep = kMfmaStep;  // keys per MFMA step
constexpr int kWaves = 4;         // prefill (one row tile per wave)

// One 16-row tile `rt` of the workgroup's waves (see the kernel below).
// LATE: the struct is read from the kernel arguments only once the first key
// loads are out (the values those need arrive preloaded in ld); otherwise
// `args` is used from the start (per-row lengths: the first loads need them).
template <int DT, int RW, int NW, bool FUSED, bool ROPE, bool RAGGED, bool LATE>
__device__ __forceinline__ void attn_mfma_tile(const Lead &ld, const AttnArgs &args, const int rt) {
  constexpr int D = kHeadDim;
  constexpr int ROWB = kHeadDim * 2;
  constexpr int VPR = ROWB / 16;
  constexpr int NPH = NW / RW;  // waves sharing a row tile
  static_assert(DT != F32, "matrix-core tiles take 16-bit storage");
  static_assert(!(LATE && RAGGED), "per-row lengths come from the struct");

  AttnArgs a;
  // the struct fields every path uses, fetched in one round of scalar loads
  auto fetch_args = [&]() {
    hoist_args(a);
    asm volatile("" ::"s"(a.scale_log2));
    if constexpr (ROPE) asm volatile("" ::"s"(a.rope_ratio));
  };
  if constexpr (!LATE) {
    a = args;
    fetch_args();
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
  const int c = lane & 15, gq = lane >> 4;
  const int split = blockIdx.x, unit = blockIdx.z;
  const int phase = wave / RW;
  const int bkv = (int)fast_div((uint32_t)unit, ld.div_Hkv), hk = unit - bkv * ld.Hkv;
  const int k0 = split * ld.chunk;
  const RowSpan sp = row_span<RAGGED>(a, bkv, ld.L, ld.causal_base, ld.new_base);
  const int kspan = min(k0 + ld.chunk, sp.L);
  const size_t head = (size_t)unit;  // bkv * Hkv + hk
  char *kc = ld.k + head * ld.S_max * ROWB;
  char *vc = ld.v + head * ld.S_max * ROWB;
  const int nb0 = max(k0, sp.new_base);

  // ---- the wave's first step goes out before anything else is computed
  // when every row of the tile sees all its keys (a causal row sees at least
  // keys 0 .. causal_base) and none of them is new
  const int kstride = NPH * kStep;
  int s0 = k0 + phase * kStep;
  u32x4 kA[2][2], kB[2][2];
  u32x2 vA[8], vB[8];
  // K: tile t, dims chunk kk -> key s + 16t + c, 16 bytes at dims 8gq + 32kk
  // V: lane's 8 keys s + {4gq + j (j < 4), 16 + 4gq + j - 4}, bytes [8c, 8c + 8)
  auto load_whole = [&](int s, u32x4 (&ka)[2][2], u32x2 (&vv)[8]) {
    // a uniform base plus a per-lane 32-bit offset: scalar address math
    const char *kb = kc + (size_t)s * ROWB;
    const char *vb = vc + (size_t)s * ROWB;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        ka[t][kk] = load16(kb + (uint32_t)((16 * t + c) * ROWB + gq * 16 + kk * 64));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kr = (j < 4) ? 4 * gq + j : 16 + 4 * gq + j - 4;
      vv[j] = *reinterpret_cast<const u32x2 *>(vb + (uint32_t)(kr * ROWB + c * 8));
    }
  };
  // only the waves whose steps hold new rows take them; the one holding the
  // first of them writes them into the cache
  bool takes_new = false, store_new = false;
  if (FUSED && kspan > nb0) {
    const int st0 = (nb0 - k0) / kStep, st1 = (kspan - 1 - k0) / kStep;
    takes_new = st0 % NPH == phase || st1 % NPH == phase;
    store_new = rt == 0 && st0 % NPH == phase;
  }
  // ---- this lane's query row. Without new rows its loads go out before the
  // first key loads (measured: 5-row cross attention 7.25 -> 7.08 us); the
  // fused kernels keep them after (measured slower the other way round),
  // except with rotary work: that waits for the query and the new rows, and
  // vector loads complete in issue order, so behind the key loads it would
  // start only once they had all landed, instead of under their latency.
  constexpr bool kSmallFirst = !FUSED || ROPE;
  const int grow = rt * kRows + c;
  bool active = false;
  RowId r{0, 0, 0};
  auto number_row = [&]() {
    active = grow < a.G;
    if (active) r = row_id(a, bkv, hk, grow);
  };
  if constexpr (!LATE) number_row();
  u32x4 qraw[2] = {u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};
  auto load_q = [&]() {
    if (active) {
      const char *qrow = static_cast<const char *>(a.q) + out_row(a, r) * 2;
      qraw[0] = load16(qrow + gq * 16);
      qraw[1] = load16(qrow + 64 + gq * 16);
    }
  };
  if constexpr (kSmallFirst && !LATE) load_q();

  // ---- new rows (decode_step_self): a wave that needs them loads them,
  // rotates them (exactly as kv_append does) while its key loads are in
  // flight, and keeps them in its own slice of LDS, so no barrier is needed;
  // the one holding the first of them writes them into the cache after its
  // key loop.
  // Lane l takes chunk pair l % 4 of new row l / 4 (N <= 16 rows: one each).
  constexpr int kNewSlice = 2 * kMaxFusedRows * VPR;  // K rows, then V rows
  __shared__ u32x4 s_new[FUSED ? NW * kNewSlice : 1];
  u32x4 *my_new = s_new + (FUSED ? wave * kNewSlice : 0);
  const int new_items = takes_new ? (kspan - nb0) * (VPR / 2) : 0;  // uniform
  PairChunks nw{};
  auto load_new = [&]() {
    if (lane < new_items) {
      const char *krow = static_cast<const char *>(a.k_new) +
                         (head * a.T_new + (nb0 - sp.new_base) + lane / 4) * ROWB;
      const char *vrow = static_cast<const char *>(a.v_new) +
                         (head * a.T_new + (nb0 - sp.new_base) + lane / 4) * ROWB;
      const int j = lane % 4;
      nw.klo = load16(krow + j * 16);
      nw.khi = load16(krow + 64 + j * 16);
      nw.vlo = load16(vrow + j * 16);
      nw.vhi = load16(vrow + 64 + j * 16);
    }
  };
  if constexpr (FUSED && kSmallFirst && !LATE) load_new();

  const int kend_lo = min(kspan, (sp.causal_base < 0) ? sp.L : sp.causal_base + 1);
  const bool early = s0 + kStep <= kend_lo && (!FUSED || s0 + kStep <= nb0);  // uniform
  if (early) load_whole(s0, kA, vA);
  if constexpr (LATE) {  // the struct, then what needs it
    a = lead_struct();
    fetch_args();
    number_row();
    if constexpr (kSmallFirst) load_q();
    if constexpr (FUSED && kSmallFirst) load_new();
  }

  // ---- the keys this lane's row sees
  const int lim = active ? ((sp.causal_base < 0) ? sp.L : sp.causal_base + r.i + 1) : 0;
  // (lanes 16 apart hold the same row: the 16 rows' bound is a max over
  // lanes 0 .. 15, taken from lane 0)
  const int kend = __builtin_amdgcn_readlane(min(kspan, (int)lanes_max<16>((float)lim)), 0);
  // below lim_lo every row of the wave sees every key
  const int lim_lo =
      __builtin_amdgcn_readlane(-(int)lanes_max<16>(-(float)(active ? lim : INT_MAX / 2)), 0);

  // ---- query operand: dims [8gq, +8) and [32 + 8gq, +8) of the row; a rotary
  // pair (i, i + 32) sits in one lane
  if constexpr (!kSmallFirst) load_q();

  float m = -INFINITY, lsum = 0.f;
  f32x4 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 qhi[2], qlo[2];  // the query operand, set once the q loads are back

  if constexpr (FUSED && !kSmallFirst) load_new();

  // One 32-key step: its loads, then its scores, softmax update and P.V.
  auto load_step = [&](int s0, u32x4 (&ka)[2][2], u32x2 (&vv)[8]) {
    // K: tile t, dims chunk kk -> key s0 + 16t + c, 16 bytes at dims 8gq + 32kk
    // V: lane's 8 keys s0 + {4gq + j (j < 4), 16 + 4gq + j - 4}, bytes [8c, 8c + 8)
    if (s0 + kStep <= kend && (!FUSED || s0 + kStep <= nb0)) {  // whole step cached
      load_whole(s0, ka, vv);
      return;
    }
    // Part of the step lies past kend or holds new rows. Every lane still
    // loads, its key clamped to the step's last cached key (row 0 if there is
    // none), so these are plain loads like the ones above: a masked load
    // behind a zeroed register would make the compiler wait for earlier loads
    // first. compute_step replaces or masks what lies outside.
    const int kcap = max(FUSED ? min(kend, nb0) - 1 : kend - 1, 0);
    const int kbase = min(s0, kcap);  // uniform; offsets from it are in [0, 32 rows)
    const char *kb = kc + (size_t)kbase * ROWB;
    const char *vb = vc + (size_t)kbase * ROWB;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t row = (uint32_t)(min(s0 + 16 * t + c, kcap) - kbase) * ROWB;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) ka[t][kk] = load16(kb + row + gq * 16 + kk * 64);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = s0 + ((j < 4) ? 4 * gq + j : 16 + 4 * gq + j - 4);
      vv[j] = *reinterpret_cast<const u32x2 *>(vb + (uint32_t)(min(key, kcap) - kbase) * ROWB + c * 8);
    }
  };
  auto compute_step = [&](int s0, u32x4 (&ka)[2][2], u32x2 (&vv)[8]) {
    if (!(s0 + kStep <= kend && (!FUSED || s0 + kStep <= nb0))) {  // uniform
      // keys past kend: their scores are masked below, and their values are
      // zeroed so that p = 0 meets no Inf or NaN of an unwritten row
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = s0 + ((j < 4) ? 4 * gq + j : 16 + 4 * gq + j - 4);
        if (key >= kend) vv[j] = u32x2{0, 0};
      }
      if constexpr (FUSED && ROPE) {
        // the step's new rows come from the wave's LDS slice: every lane reads
        // at its row clamped into the slice and selects. In the rotary tile a
        // read inside a per-lane branch waited for its own round trip, one
        // after another: about 1 us for the step holding the new row of a GQA
        // decode step (with the new-key angles computed only by the waves that
        // take new rows, below: 6.70 -> 6.47 us at length 768). The other
        // fused tiles keep the reads in the branch (the 5-draft step at length
        // 448 measured 6.01 against 6.28 us the other way).
        u32x4 nk[2][2];
        u32x4 nvr[8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r = min(max(s0 + 16 * t + c - nb0, 0), kMaxFusedRows - 1);
          nk[t][0] = my_new[r * VPR + gq];
          nk[t][1] = my_new[r * VPR + gq + VPR / 2];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = s0 + ((j < 4) ? 4 * gq + j : 16 + 4 * gq + j - 4);
          const int r = min(max(key - nb0, 0), kMaxFusedRows - 1);
          nvr[j] = my_new[(kMaxFusedRows + r) * VPR + c / 2];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int key = s0 + 16 * t + c;
          const bool fresh = key < kend && key >= nb0;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) ka[t][kk][i] = fresh ? nk[t][kk][i] : ka[t][kk][i];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = s0 + ((j < 4) ? 4 * gq + j : 16 + 4 * gq + j - 4);
          const bool fresh = key < kend && key >= nb0;
          const u32x2 nv2 = (c & 1) ? u32x2{nvr[j][2], nvr[j][3]} : u32x2{nvr[j][0], nvr[j][1]};
          vv[j] = fresh ? nv2 : vv[j];
        }
      } else if constexpr (FUSED) {  // the step's new rows come from the wave's LDS slice
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int key = s0 + 16 * t + c;
          if (key < kend && key >= nb0) {
            ka[t][0] = my_new[(key - nb0) * VPR + gq];
            ka[t][1] = my_new[(key - nb0) * VPR + gq + VPR / 2];
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = s0 + ((j < 4) ? 4 * gq + j : 16 + 4 * gq + j - 4);
          if (key < kend && key >= nb0) {
            const u32x4 row = my_new[(kMaxFusedRows + key - nb0) * VPR + c / 2];
            vv[j] = (c & 1) ? u32x2{row[2], row[3]} : u32x2{row[0], row[1]};
          }
        }
      }
    }
    // scores S^T: st[t][i] = q_row . k_(s0 + 16t + 4gq + i)
    f32x4 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = mfma<DT>(ka[t][0], qhi[0], f32x4{0.f, 0.f, 0.f, 0.f});
      st[t] = mfma<DT>(ka[t][1], qhi[1], st[t]);
      if constexpr (ROPE) {
        st[t] = mfma<DT>(ka[t][0], qlo[0], st[t]);
        st[t] = mfma<DT>(ka[t][1], qlo[1], st[t]);
      }
    }
    float sc[8];
    float mt = -INFINITY;
    if (s0 + kStep <= lim_lo && s0 + kStep <= kend) {  // every row sees every key
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sc[j] = st[j >> 2][j & 3] * a.scale_log2;
        mt = fmaxf(mt, sc[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = j >> 2, i = j & 3;
        const int key = s0 + 16 * t + 4 * gq + i;
        sc[j] = (key < lim && key < kend) ? st[t][i] * a.scale_log2 : -INFINITY;
        mt = fmaxf(mt, sc[j]);
      }
    }
    mt = groups_max<16>(mt);  // the row's 32 keys sit in lanes c, c+16, c+32, c+48
    // lazy reference, as online_update: m moves only when a score passes it
    // by more than kLazySoftmax; o and l are rescaled only when a row moved
    const bool move = mt > m + kLazySoftmax;
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float mn = move ? mt : m;
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] *= alpha;
      lsum *= alpha;
      m = mn;
    }
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[j] - m);
      ps += p[j];
    }
    lsum += ps;
    u32x4 phi, plo;
    split_hi_lo<DT>(p, phi, plo);
    // V^T rows 4c + t: element t of each of the 8 key chunks
    const u32x4 va[4] = {
        u32x4{pair16<0>(vv[0], vv[1]), pair16<0>(vv[2], vv[3]), pair16<0>(vv[4], vv[5]), pair16<0>(vv[6], vv[7])},
        u32x4{pair16<1>(vv[0], vv[1]), pair16<1>(vv[2], vv[3]), pair16<1>(vv[4], vv[5]), pair16<1>(vv[6], vv[7])},
        u32x4{pair16<2>(vv[0], vv[1]), pair16<2>(vv[2], vv[3]), pair16<2>(vv[4], vv[5]), pair16<2>(vv[6], vv[7])},
        u32x4{pair16<3>(vv[0], vv[1]), pair16<3>(vv[2], vv[3]), pair16<3>(vv[4], vv[5]), pair16<3>(vv[6], vv[7])}};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      o[t] = mfma<DT>(va[t], phi, o[t]);
      o[t] = mfma<DT>(va[t], plo, o[t]);
    }
  };

  // ---- otherwise the wave's first step goes out now, into the second
  // buffer: loaded into the first, whose early loads the compiler cannot rule
  // out on this path, it waited for every load issued so far (the query's and
  // the new rows' included) before issuing these. The fused rotary kernel
  // keeps the first buffer (measured faster there: 6.72 against 6.84 us for
  // the GQA step at length 768; elsewhere the second buffer wins, e.g. the
  // 5-draft step at length 448, 6.33 -> 6.01 us).
  constexpr bool kFirstB = !(FUSED && ROPE);
  const bool first_b = kFirstB && !early;  // uniform
  if (!early && s0 < kend) {
    if (kFirstB) load_step(s0, kB, vB);
    else load_step(s0, kA, vA);
  }

  // ---- cos / sin of the new rows' keys and of the query row: no memory
  // access, so they are all computed while the loads above are in flight (the
  // scheduling barrier keeps the compiler from moving the first use of a
  // loaded value, and so the wait for it, in between)
  double ncs[ROPE && FUSED ? 8 : 1], nsn[ROPE && FUSED ? 8 : 1];  // new keys: fp64
  float qc[ROPE ? 8 : 1], qs[ROPE ? 8 : 1];
  // Fused steps of up to 16 rows (new rows where the queries are), and one
  // query without new rows: every position the tile needs lies in
  // causal_base + [0, N), so the wave computes the fp32 cos / sin of those
  // N x 32 pairs once, one pair per lane at a time, into its own LDS slice
  // (position p: cos in slots 64p .. 64p + 31, sin in the next 32), and each
  // lane reads its query's values back. The new keys are then rotated one
  // pair per lane in the wave's LDS slice (pair_rot below), each with its
  // own fp64 cos / sin. (Without new rows and N > 1 a lane's own 8 query
  // pairs cost about as much as its share of the table: measured 4.72
  // against 4.91 us for 5 queries at length 64.)
  constexpr int kRopeSlice = kMaxFusedRows * 64;
  __shared__ __attribute__((aligned(16))) float s_rope[(ROPE && RW == 1) ? NW * kRopeSlice : 1];
  bool shared_cs = false;
  if constexpr (ROPE && RW == 1)
    shared_cs = FUSED ? (a.N <= kMaxFusedRows && sp.new_base == sp.causal_base) : a.N == 1;  // uniform
  // pair_rot below: the exact angle of this lane's first new-key pair, here,
  // under the loads' latency (it needs only the position and the pair)
  double th_pair = 0.0, c_pair = 1.0, s_pair = 0.0;
  if (shared_cs) {
    if constexpr (ROPE && RW == 1 && FUSED) {
      if (new_items > 0) {  // uniform: only the waves that take new rows rotate them
        th_pair = rope_theta_at(a.rope_theta, lane & 31);  // exact, as kv_append's
        if (lane < new_items / (VPR / 2) * 32) rope_angle_cs64(nb0 + lane / 32, th_pair, c_pair, s_pair);
      }
    }
    if constexpr (ROPE && RW == 1) {
      float *tab = s_rope + wave * kRopeSlice;
      for (int idx = lane; idx < a.N * 32; idx += 64) {
        const int pos = sp.causal_base + idx / 32, slot = (idx / 32) * 64 + idx % 32;
        float cl, sl;
        rope_cos_sin_pair<8>(pos, idx % 32, RopeStep{a.rope_ratio}, cl, sl);
        tab[slot] = cl;
        tab[slot + 32] = sl;
      }
      asm volatile("" ::: "memory");  // the slice is written before the wave reads it
      const float *qt = tab + r.i * 64 + 8 * gq;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qc[e] = qt[e];
        qs[e] = qt[32 + e];
      }
    }
  } else {
    if constexpr (ROPE && FUSED) {
      double thn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) thn[e] = rope_theta_at(a.rope_theta, (lane % 4) * 8 + e);
      if (lane < new_items) rope_cos_sin_run64<8>(nb0 + lane / 4, thn, ncs, nsn);
    }
    if constexpr (ROPE)
      rope_cos_sin_run<8>(sp.causal_base + r.i, gq * 8, RopeStep{a.rope_ratio}, qc, qs);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- the new rows into the wave's slice, keys rotated as kv_append
  // rotates them: per lane (8 pairs each) off the shared table, else one pair
  // per lane in the slice, then stored from there
  if constexpr (FUSED) {
    const bool pair_rot = ROPE && shared_cs;  // uniform
    if (lane < new_items) {
      const int rr = lane / 4, j = lane % 4;
      if constexpr (ROPE) {
        if (!pair_rot) rotate_key_pair_cs<DT>(nw.klo, nw.khi, ncs, nsn);
      }
      my_new[rr * VPR + j] = nw.klo;
      my_new[rr * VPR + j + VPR / 2] = nw.khi;
      my_new[(kMaxFusedRows + rr) * VPR + j] = nw.vlo;
      my_new[(kMaxFusedRows + rr) * VPR + j + VPR / 2] = nw.vhi;
    }
    asm volatile("" ::: "memory");  // the slice is written before the wave reads it
    if constexpr (ROPE) {
      if (pair_rot && new_items > 0) {  // uniform
        const int rows = new_items / (VPR / 2);
        for (int item = lane; item < rows * 32; item += 64) {  // pair item % 32 == lane % 32
          const int rr = item / 32, pr = item % 32;
          double c64 = c_pair, s64 = s_pair;
          if (item != lane) rope_angle_cs64(nb0 + rr, th_pair, c64, s64);
          uint16_t *kr = reinterpret_cast<uint16_t *>(my_new + rr * VPR);
          float lo = widen16<DT>(kr[pr]), hi = widen16<DT>(kr[pr + kHeadDim / 2]);
          rotate_elem64<DT>(lo, hi, c64, s64);
          const uint32_t w = pack2<DT>(lo, hi);
          kr[pr] = (uint16_t)w;
          kr[pr + kHeadDim / 2] = (uint16_t)(w >> 16);
        }
        asm volatile("" ::: "memory");  // rotated before the wave reads them
      }
    }
  }

  // ---- query operand (rotated in fp32, fed as a high and a low part)
  if constexpr (ROPE) {
    float x0[8], x1[8];
    unpack16<DT>(qraw[0], x0);
    unpack16<DT>(qraw[1], x1);
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_rotate(x0[e], x1[e], qc[e], qs[e]);
    split_hi_lo<DT>(x0, qhi[0], qlo[0]);
    split_hi_lo<DT>(x1, qhi[1], qlo[1]);
  } else {
    qhi[0] = qraw[0];
    qhi[1] = qraw[1];
    qlo[0] = qlo[1] = u32x4{0, 0, 0, 0};
  }

  {
    // the next step's loads go out before this step's math (two register
    // buffers in turn; three steps ahead measured no faster in prefill)
    // (a wave whose first step is in the second buffer enters at its half)
    bool skip_a = first_b;  // uniform
    while (s0 < kend) {
      if (!skip_a) {
        if (s0 + kstride < kend) load_step(s0 + kstride, kB, vB);
        compute_step(s0, kA, vA);
        s0 += kstride;
        if (s0 >= kend) break;
      }
      skip_a = false;
      if (s0 + kstride < kend) load_step(s0 + kstride, kA, vA);
      compute_step(s0, kB, vB);
      s0 += kstride;
    }
  }
  lsum = groups_sum<16>(lsum);  // the row's keys were spread over the 4 lane groups

  // ---- the new rows into the cache, from the wave's slice, after the key
  // loop (a store counts in vmcnt with the loads: issued before the loop,
  // every wait for a key load there would wait for it too)
  if constexpr (FUSED) {
    if (store_new && lane < new_items) {
      const int rr = lane / 4, j = lane % 4, pos = nb0 + rr;
      const PairChunks c{my_new[rr * VPR + j], my_new[rr * VPR + j + VPR / 2],
                         my_new[(kMaxFusedRows + rr) * VPR + j],
                         my_new[(kMaxFusedRows + rr) * VPR + j + VPR / 2]};
      store_pair<DT>(kc + (size_t)pos * ROWB, vc + (size_t)pos * ROWB, j, c);
    }
  }

  // ---- lane l holds O[row c][16gq + 4i + t] = o[t][i]; merge the phases
  // that shared the row tile, then write the rows or publish the partial
  constexpr int kSmem = (RW == NW) ? 1 : NW * kRows * (D + 2);
  __shared__ __attribute__((aligned(16))) float smem[kSmem];
  const size_t tile_id = (size_t)unit * a.row_tiles + blockIdx.y;
  if constexpr (RW == NW) {
    // one wave per row tile, no split (the plan guarantees it)
    if (active) {
      const float inv = 1.f / lsum;
      float *orow = a.out + out_row(a, r) + 16 * gq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int t = 0; t < 4; ++t) store_f32(orow + 4 * i + t, o[t][i] * inv);
      }
    }
    return;
  } else {
    float *sm_o = smem;                        // [phase][row][D]
    float *sm_m = smem + NW * kRows * D;   // [phase][row]
    float *sm_l = sm_m + NW * kRows;       // [phase][row]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int t = 0; t < 4; ++t) sm_o[(phase * kRows + c) * D + 16 * gq + 4 * i + t] = o[t][i];
    }
    if (gq == 0) {
      sm_m[phase * kRows + c] = m;
      sm_l[phase * kRows + c] = lsum;
    }
    __syncthreads();
    const int g0 = blockIdx.y * kRows;
    const int gcount = min(kRows, a.G - g0);
    float *part = a.ws_part + (tile_id * a.splits + split) * kRows * kPStride;
    for (int idx = threadIdx.x; idx < gcount * D; idx += blockDim.x) {
      const int g = idx / D, d = idx % D;
      float mw[NPH], lw[NPH];
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NPH; ++w) {
        mw[w] = sm_m[w * kRows + g];
        lw[w] = sm_l[w * kRows + g];
        M = fmaxf(M, mw[w]);
      }
      // no branches: a phase with no keys (m = -inf) contributes zeros
      float Ls = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < NPH; ++w) {
        const bool ok = mw[w] != -INFINITY;
        const float ow = sm_o[(w * kRows + g) * D + d];
        const float f = ok ? __builtin_amdgcn_exp2f(mw[w] - M) : 0.f;
        Ls = fmaf(ok ? lw[w] : 0.f, f, Ls);
        O = fmaf(ok ? ow : 0.f, f, O);
      }
      if (a.splits == 1) {
        store_f32(a.out + out_row(a, row_id(a, bkv, hk, g0 + g)) + d, O * __builtin_amdgcn_rcpf(Ls));
      } else {
        publish(part + g * kPStride + d, O);
        if (d == 0) {
          publish(part + g * kPStride + D, M);
          publish(part + g * kPStride + D + 1, Ls);
        }
      }
    }
    if (a.splits == 1) return;
    merge_splits<kRows>(a, tile_id, g0, gcount, bkv, hk, NW);
  }
}

template <int DT, int RW, int NW, bool FUSED, bool ROPE, bool RAGGED>
__global__ __launch_bounds__(64 * NW) void attn_mfma_kernel(KVD_LEAD_PARAMS, AttnArgs a) {
  const Lead ld = KVD_LEAD;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (RW == NW && !FUSED) {
    if (a.pair) {  // causal prefill: tile t and its complement T - 1 - t
      const int T = (a.G + kRows - 1) / kRows;
      const int t = blockIdx.y * RW + wave;
      if (t >= (T + 1) / 2) return;  // no barrier follows in this mode
      attn_mfma_tile<DT, RW, NW, FUSED, ROPE, RAGGED, false>(ld, a, t);
      if (T - 1 - t > t) attn_mfma_tile<DT, RW, NW, FUSED, ROPE, RAGGED, false>(ld, a, T - 1 - t);
      return;
    }
    attn_mfma_tile<DT, RW, NW, FUSED, ROPE, RAGGED, false>(ld, a, blockIdx.y * RW + wave % RW);
  } else {
    attn_mfma_tile<DT, RW, NW, FUSED, ROPE, RAGGED, !RAGGED>(ld, a, blockIdx.y * RW + wave % RW);
  }
}

template <int DT, int RW, int NW, bool RAGGED>
void launch_rwr(const AttnArgs &a, dim3 grid, hipStream_t s) {
  const bool fused = a.k_new != nullptr, rope = a.rope_base > 0.f;
  const dim3 block(64 * NW);
  if constexpr (RW == 1 && NW == 8) {
    // rotary tiles always run on 4 waves (launch_dt): their per-wave LDS
    // tables would not fit 8
    (void)rope;
    if (fused) launch_lead(attn_mfma_kernel<DT, RW, NW, true, false, RAGGED>, grid, block, s, a);
    else launch_lead(attn_mfma_kernel<DT, RW, NW, false, false, RAGGED>, grid, block, s, a);
  } else if (fused) {
    if (rope) launch_lead(attn_mfma_kernel<DT, RW, NW, true, true, RAGGED>, grid, block, s, a);
    else launch_lead(attn_mfma_kernel<DT, RW, NW, true, false, RAGGED>, grid, block, s, a);
  } else {
    if (rope) launch_lead(attn_mfma_kernel<DT, RW, NW, false, true, RAGGED>, grid, block, s, a);
    else launch_lead(attn_mfma_kernel<DT, RW, NW, false, false, RAGGED>, grid, block, s, a);
  }
}

template <int DT, int RW, int NW>
void launch_rw(const AttnArgs &a, dim3 grid, hipStream_t s) {
  if (a.lens) launch_rwr<DT, RW, NW, true>(a, grid, s);
  else launch_rwr<DT, RW, NW, false>(a, grid, s);
}

// prefill tiles on 4 waves; shared tiles on 4 or 8 (the plan's a.waves;
// rotary tiles on 4)
template <int DT>
void launch_dt(const AttnArgs &a, dim3 grid, hipStream_t s) {
  if (a.rw == kWaves) launch_rw<DT, kWaves, kWaves>(a, grid, s);
  else if (a.waves == 8 && !(a.rope_base > 0.f)) launch_rw<DT, 1, 8>(a, grid, s);
  else launch_rw<DT, 1, 4>(a, grid, s);
}

}  // namespace

hipError_t launch_attn_mfma(int dtype, const AttnArgs &a, hipStream_t s) {
  if (a.rw == kWaves && !a.k_new) return launch_prefill(dtype, a, s);
  const dim3 grid(a.splits, a.row_tiles, a.Bkv * a.Hkv);
  if (dtype == F16) launch_dt<F16>(a, grid, s);
  else launch_dt<BF16>(a, grid, s);
  return hipGetLastError();
}

}  // namespace kvd
