// Internal interface between the C-ABI entry points (validation, planning)
// and the kernel launchers. Nothing here is exported.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct kvd_cache;  // the C ABI's cache descriptor (kvdecode.h)

namespace kvd {

enum DType { F32 = 0, F16 = 1, BF16 = 2 };  // same values as enum kvd_dtype

constexpr int kHeadDim = 64;

// Status values kernels store in a caller's dev_status word (the values of
// KVD_ERR_SHAPE and KVD_ERR_CAPACITY).
constexpr int kStatusBadShape = -2;
constexpr int kStatusCapacity = -4;

// Arrival counters at the start of every workspace (one per merged tile),
// each on a 128-byte cache line of its own: counters that share a line make
// the arrivals of different tiles wait on one another (measured on the
// 20-head cross attention: 7.65 -> 7.15 us).
constexpr int kMaxCounters = 4096;
constexpr int kCounterStride = 32;  // uint32 words from one counter to the next
// decode_step_self: new rows appended inside the attention launch (more are
// appended by a separate kv_append launch first).
constexpr int kMaxFusedRows = 16;
constexpr int kMaxSplits = 64;  // key splits per tile: the merge gives each split one lane
// verify_accept: (value, index) pairs one batch row may stage for its merge.
constexpr int kMaxVerifyChunks = 512;  // 2048-logit chunks per row (8 keys per lane in the merge)

// Rotary angle per pair, theta_i = base^(-2i/D) for i < D/2, as the host's C
// library pow gives it in fp64, carried in a form a kernel rebuilds in
// registers (no table in memory): with r = pow(base, -2/D) and pw[k] = r^(2^k)
// by repeated squaring, theta'_i is the product of pw[k] over the set bits k
// of i, multiplied in ascending k (IEEE fp64 products, the same on host and
// device), and delta_i = bits(theta_i) - bits(theta'_i) is a small signed
// count of ulps (|delta_i| <= 24 for bases 1e-3 .. 3.4e38), packed four to a
// word; theta_i's bits are theta'_i's plus delta_i.
struct RopeTheta {
  double pw[5];
  uint32_t delta[kHeadDim / 8];
};

struct AppendArgs {
  void *k_cache, *v_cache;       // [B][H][S_max][D]
  const void *k_new, *v_new;     // [B][H][T][D]
  int B, H, S_max, T, pos;
  const int32_t *pos_rows;       // [B] per-row positions (ragged batch), or null: pos for all
  int32_t *dev_status;           // a row outside the cache is skipped and flagged here, or null
  float rope_base;               // > 0: rotate keys at pos + t
  RopeTheta rope_theta;          // exact theta_i for stored keys, when rope_base > 0
};

struct ReorderArgs {
  void *k_cache, *v_cache;       // [B][H][S_max][D]
  const int32_t *parent;         // [B]
  int32_t *dev_status;           // nullable
  int B, H, S_max, len;
};

// One attention launch. A "unit" is one (cache row, kv head) pair; its query
// rows are every (b, h, i) that reads it, numbered g = (bl * group + j) * N + i
// with bl the batch row within the unit (0 unless the cache is shared),
// j the head within the group and i the query.
// Division by a divisor fixed for a launch, as a multiply-high (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// for 1 <= d < 2^31, s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1,
// n / d = (umulhi(n, m) + n) >> s for every 0 <= n < 2^31 (the sum stays below
// 2^32). A few instructions where a runtime division takes about twenty.
struct FastDiv {
  uint32_t m, s;
};
inline FastDiv make_fast_div(uint32_t d) {
  uint32_t s = 0;
  while (((uint64_t)1 << s) < d) ++s;
  return FastDiv{(uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << s) - d)) / d + 1), s};
}

struct AttnArgs {
  const void *q;                 // [B][Hq][N][D]
  void *k, *v;                   // [Bkv][Hkv][S_max][D]
  const void *k_new, *v_new;     // [Bkv][Hkv][T_new][D] rows appended in this launch, or null
  float *out;                    // [B][Hq][N][D]
  float *ws_part;                // partial (o, m, l) per split
  uint32_t *ws_count;            // arrival counters, one per (unit, row tile), kCounterStride apart
  int B, Hq, N, Bkv, Hkv, group, S_max;
  FastDiv div_N, div_group;      // division by N and by group (query row numbering)
  int G;                         // query rows per unit
  int L;                         // keys: len (self) or frames (cross)
  int causal_base;               // self: len - N; cross: -1 (no mask)
  int new_base, T_new;           // new rows sit at [new_base, new_base + T_new); INT_MAX: none
  const int32_t *lens;           // [Bkv] per-row len (ragged self attention; L is then the
                                 // planned maximum), or null
  int32_t *dev_status;           // a len outside [N, L] is clamped and flagged here, or null
  const void *k_src, *v_src;     // beam step: cached rows are read from beam parent[b] here
  const int32_t *parent;         // [Bkv] beam step parents (k, v are then the destination), or null
  float scale_log2;              // scale * log2(e)
  float rope_base;               // > 0: rotate q at causal_base + i (and new keys)
  double rope_ratio;             // 2^(-2 log2(base) / D): queries turn pair i by theta_i = rope_ratio^i
  RopeTheta rope_theta;          // new keys: the exact theta_i (as kv_append stores them)
  // plan
  int chunk;                     // keys per workgroup
  int splits;                    // workgroups per (unit, row tile)
  int row_tiles;                 // ceil(G / rows per tile)
  int waves;                     // waves per workgroup
  int gm;                        // rows per tile (template bucket)
  int mfma;                      // 1: matrix-core tile kernel (blocks of queries)
  int rw;                        // matrix-core kernel: 16-row tiles per workgroup (1 or 4)
  int pair;                      // rw = 4, causal: each wave takes tiles t and T - 1 - t
};

struct VerifyArgs {
  const void *logits;            // [B][R][V]
  int dtype;
  const int32_t *draft;          // [B][N]
  int32_t *argmax_out;           // [B][R] or null
  int32_t *accept_len, *next_token;
  const uint32_t *suppress;      // [ceil(V / 32)] bit t: token t at -inf on every row, or null
  const uint32_t *suppress_first;  // the same for row 0 of each batch row, or null
  uint64_t *ws_key;              // [B][R][chunks]
  uint32_t *ws_count;            // [B], kCounterStride apart
  int B, R, V, N;
  int chunk, chunks;
};

// Plan forced by kvd_set_plan_override (a testing hook): mfma -1 none, 0 keep
// 16-bit caches on the streaming kernel; waves, chunk 0: as planned.
struct PlanOverride {
  int mfma, waves, chunk;
};
PlanOverride plan_override();
void set_plan_override(PlanOverride o);

// Attention planning shared by the entry points and the workspace-size query.
struct AttnPlan {
  int gm, row_tiles, chunk, splits, waves, mfma, rw;
  size_t part_floats, counters;
};
AttnPlan plan_attn(int dtype, int units, int G, int N, int L, bool rope, bool allow_mfma = true);

void plan_verify(int B, int R, int V, int &chunk, int &chunks);

// Events a caller asked the next launch of this thread to record (kernel
// begin / end); taken and cleared by that launch.
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTiming take_launch_timing();

// Every kernel of the library is launched through here.
template <typename... Args>
inline void launch_kernel(void (*kernel)(Args...), dim3 grid, dim3 block, hipStream_t s,
                          Args... args) {
  void *argv[] = {static_cast<void *>(&args)...};
  const LaunchTiming t = take_launch_timing();
  if (t.start || t.stop)
    (void)hipExtLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, 0, s,
                             t.start, t.stop, 0);
  else
    (void)hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, 0, s);
}

// decode_step_self's work: validation and planning (all on the host before
// any HIP call) and, unless check_only, the launches on `stream`.
int step_self(const void *q, const void *k_new, const void *v_new, int32_t Hq, int32_t N,
              const ::kvd_cache *cache, int32_t len, float scale, float rope_base, float *out,
              void *ws, size_t ws_bytes, void *stream, bool check_only);

hipError_t launch_append(int dtype, const AppendArgs &a, hipStream_t s);
hipError_t launch_reorder(int dtype, const ReorderArgs &a, hipStream_t s);
hipError_t launch_attn(int dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_mfma(int dtype, const AttnArgs &a, hipStream_t s);
// Prefill-sized blocks of queries (a matrix-core plan of four 16-row tiles
// per workgroup, no new rows): K/V staged through LDS once per workgroup.
hipError_t launch_prefill(int dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_verify(const VerifyArgs &a, hipStream_t s);

// Beam-search candidate scoring.
constexpr int kMaxBeamWidth = 16;                    // beams per audio row
constexpr int kBeamRec = 2 + 2 * (kMaxBeamWidth + 1);  // words per chunk record
constexpr int kMaxBeamEntries = 512;                 // chunk entries merged per beam (8 per lane)
struct BeamArgs {
  const void *logits;            // [B][K][V]
  int dtype;
  const float *sum_logprobs;     // [B][K]
  int32_t *parent, *token;       // [B][K]
  float *score;                  // [B][K]
  int32_t *fin_count;            // [B]
  int32_t *fin_parent;           // [B][K]
  float *fin_score;              // [B][K]
  uint32_t *ws_count;            // [B], kCounterStride apart
  uint32_t *ws_rec;              // [B][K][chunks][kBeamRec]
  int B, K, V, eot, chunks;
};
int beam_chunks(int V);
hipError_t launch_beam(const BeamArgs &a, hipStream_t s);

struct ProbeArgs {
  const void *a, *b;  // buffers to read (b may be NULL)
  size_t vecs;        // 16-byte vectors read from each
  uint32_t *sink;
  int unroll;         // loads in flight per thread: 1, 2, 4, 8 or 16
  size_t blocks;      // workgroups of 256 threads; 0: one round of loads per thread
};
int probe_unroll_ok(int u);
hipError_t launch_probe(const ProbeArgs &a, hipStream_t s);

}  // namespace kvd
