// C-ABI entry points: argument validation (all of it before any HIP call),
// launch planning, and status codes. The operations are defined in
// include/kvdecode.h.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "kvd_internal.hpp"
#include "kvdecode.h"

using kvd::AttnArgs;
using kvd::AttnPlan;

static_assert(kvd::kStatusBadShape == KVD_ERR_SHAPE, "kernel status values");
static_assert(kvd::kStatusCapacity == KVD_ERR_CAPACITY, "kernel status values");

namespace {

bool dtype_ok(int dt) { return dt == KVD_F32 || dt == KVD_F16 || dt == KVD_BF16; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
// Aligned to its element type (logits are read one element at a time).
bool elem_aligned(const void *p, int dtype) {
  return (reinterpret_cast<uintptr_t>(p) & (dtype == KVD_F32 ? 3u : 1u)) == 0;
}

// Shared checks of a cache descriptor.
int check_cache(const kvd_cache *c) {
  if (!c) return KVD_ERR_NULL;
  if (!c->k || !c->v) return KVD_ERR_NULL;
  if (!dtype_ok(c->dtype)) return KVD_ERR_DTYPE;
  if (c->B < 1 || c->H < 1 || c->S_max < 1 || c->D != kvd::kHeadDim) return KVD_ERR_SHAPE;
  if (!aligned16(c->k) || !aligned16(c->v)) return KVD_ERR_ALIGN;
  return KVD_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? KVD_OK : KVD_ERR_LAUNCH; }

// Rotary angles theta_i = base^(-2i/D), i < D/2, each the C library's fp64
// pow of the exact exponent -2i/D ([N] "nanoVLM における技術的実装", item 2:
// rotary positions at start_pos; the RoFormer frequencies); zeros without
// rotation.
// Returns false if a correction does not fit its byte (never seen: at most
// 24 ulps for bases 1e-3 .. 3.4e38).
bool rope_theta_of(float rope_base, kvd::RopeTheta &r) {
  r = kvd::RopeTheta{};
  if (!(rope_base > 0.f)) return true;
  const double base = rope_base;
  r.pw[0] = pow(base, -2.0 / kvd::kHeadDim);
  for (int k = 1; k < 5; ++k) r.pw[k] = r.pw[k - 1] * r.pw[k - 1];
  for (int i = 0; i < kvd::kHeadDim / 2; ++i) {
    double t = 1.0;
    for (int k = 0; k < 5; ++k) t = t * (((i >> k) & 1) ? r.pw[k] : 1.0);
    const double theta = pow(base, -2.0 * i / kvd::kHeadDim);
    int64_t bt, bp;
    memcpy(&bt, &theta, 8);
    memcpy(&bp, &t, 8);
    const int64_t d = bt - bp;
    if (d < -128 || d > 127) return false;
    r.delta[i / 4] |= (uint32_t)(uint8_t)(int8_t)d << (8 * (i % 4));
  }
  return true;
}

// Every workspace starts with a fixed block of arrival counters, zero at rest
// (each kernel that counts arrivals sets its counters back to zero), so one
// workspace can serve calls with different plans: partial results of one call
// never land where another call keeps a counter.
constexpr size_t kCounterBytes = (size_t)kvd::kMaxCounters * kvd::kCounterStride * sizeof(uint32_t);

size_t attn_bytes(const AttnPlan &p) { return kCounterBytes + p.part_floats * sizeof(float); }

// Fill the plan-dependent fields and the workspace pointers.
int prepare_attn(AttnArgs &a, int dtype, void *ws, size_t ws_bytes) {
  const int units = a.Bkv * a.Hkv;
  a.div_N = kvd::make_fast_div((uint32_t)a.N);
  a.div_group = kvd::make_fast_div((uint32_t)a.group);
  // the beam step runs on the streaming kernel (it alone copies parent rows)
  const AttnPlan p = kvd::plan_attn(dtype, units, a.G, a.N, a.L, a.rope_base > 0.f, !a.parent);
  if (p.row_tiles > 65535 || units > 65535) return KVD_ERR_SHAPE;  // grid limits
  if (p.splits > kvd::kMaxSplits) return KVD_ERR_SHAPE;  // the merge gives each split one lane
  a.chunk = p.chunk;
  a.splits = p.splits;
  a.row_tiles = p.row_tiles;
  a.waves = p.waves;
  a.gm = p.gm;
  a.mfma = p.mfma;
  a.rw = p.rw;
  // Causal prefill on one tile per wave: the tiles late in a sequence walk
  // many more keys than the early ones, so each wave takes a complementary
  // pair (tile t, tile T - 1 - t; rows are ordered by head, then position),
  // which evens the waves' work and halves their number.
  a.pair = 0;
  if (p.mfma && p.rw == 4 && a.causal_base >= 0 && !a.k_new) {
    const int tiles16 = (a.G + 15) / 16;
    a.pair = 1;
    a.row_tiles = ((tiles16 + 1) / 2 + 3) / 4;
  }
  if (p.splits > 1) {
    const size_t need = attn_bytes(p);
    if (!ws) return KVD_ERR_WORKSPACE;
    if (ws_bytes < need) return KVD_ERR_WORKSPACE;
    if (!aligned16(ws)) return KVD_ERR_ALIGN;
    a.ws_count = static_cast<uint32_t *>(ws);
    a.ws_part = reinterpret_cast<float *>(static_cast<char *>(ws) + kCounterBytes);
  } else {
    a.ws_count = nullptr;
    a.ws_part = nullptr;
  }
  return KVD_OK;
}

thread_local kvd::LaunchTiming g_next_timing;

}  // namespace

kvd::LaunchTiming kvd::take_launch_timing() {
  const LaunchTiming t = g_next_timing;
  g_next_timing = LaunchTiming{};
  return t;
}

extern "C" {

int kvd_read_probe_ex(const void *a, const void *b, size_t bytes, uint32_t *sink, int32_t unroll,
                      size_t blocks, void *stream) {
  if (!a || !sink) return KVD_ERR_NULL;
  if (bytes == 0 || bytes % 16 || !kvd::probe_unroll_ok(unroll) || blocks > 65535)
    return KVD_ERR_SHAPE;
  if (!aligned16(a) || (b && !aligned16(b)) || !aligned4(sink)) return KVD_ERR_ALIGN;
  kvd::ProbeArgs p{a, b, bytes / 16, sink, unroll, blocks};
  return status_of(kvd::launch_probe(p, static_cast<hipStream_t>(stream)));
}

int kvd_read_probe(const void *a, const void *b, size_t bytes, uint32_t *sink, void *stream) {
  return kvd_read_probe_ex(a, b, bytes, sink, 4, 0, stream);
}

int kvd_set_plan_override(int32_t mfma, int32_t waves, int32_t chunk) {
  if (mfma < -1 || mfma > 1 || waves < 0 || waves > 16 || chunk < 0) return KVD_ERR_SHAPE;
  kvd::set_plan_override(kvd::PlanOverride{mfma, waves, chunk});
  return KVD_OK;
}

int kvd_time_next_launch(void *start_event, void *stop_event) {
  g_next_timing.start = static_cast<hipEvent_t>(start_event);
  g_next_timing.stop = static_cast<hipEvent_t>(stop_event);
  return KVD_OK;
}

const char *kvd_status_string(int status) {
  switch (status) {
    case KVD_OK: return "ok";
    case KVD_ERR_NULL: return "a required pointer is NULL";
    case KVD_ERR_SHAPE: return "a size is out of range or two sizes disagree";
    case KVD_ERR_DTYPE: return "unknown element type";
    case KVD_ERR_CAPACITY: return "rows beyond the cache capacity";
    case KVD_ERR_ROWS: return "logits rows must be N or N + 1";
    case KVD_ERR_WORKSPACE: return "workspace missing or too small";
    case KVD_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case KVD_ERR_LAUNCH: return "HIP launch failed";
    case KVD_ERR_SCRATCH: return "shape needs more than the static scratch array holds";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Shared by kv_append and kv_append_ragged (pos_rows non-null: per-row
// positions on the device, checked there).
int append_impl(const kvd_cache *cache, const void *k_new, const void *v_new, int32_t pos,
                const int32_t *pos_rows, int32_t *dev_status, int32_t T, float rope_base,
                void *stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (!k_new || !v_new) return KVD_ERR_NULL;
  if (T < 1 || pos < 0 || !(rope_base >= 0.f) || isinf(rope_base)) return KVD_ERR_SHAPE;
  if ((int64_t)pos + T > cache->S_max) return KVD_ERR_CAPACITY;
  if (!aligned16(k_new) || !aligned16(v_new)) return KVD_ERR_ALIGN;
  if ((pos_rows && !aligned4(pos_rows)) || (dev_status && !aligned4(dev_status)))
    return KVD_ERR_ALIGN;
  kvd::AppendArgs a{};
  a.pos_rows = pos_rows;
  a.dev_status = dev_status;
  a.k_cache = cache->k;
  a.v_cache = cache->v;
  a.k_new = k_new;
  a.v_new = v_new;
  a.B = cache->B;
  a.H = cache->H;
  a.S_max = cache->S_max;
  a.T = T;
  a.pos = pos;
  a.rope_base = rope_base;
  if (!rope_theta_of(rope_base, a.rope_theta)) return KVD_ERR_SHAPE;
  return status_of(kvd::launch_append(cache->dtype, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int kv_append(const kvd_cache *cache, const void *k_new, const void *v_new, int32_t pos,
              int32_t T, float rope_base, void *stream) {
  return append_impl(cache, k_new, v_new, pos, nullptr, nullptr, T, rope_base, stream);
}

int kv_append_ragged(const kvd_cache *cache, const void *k_new, const void *v_new,
                     const int32_t *pos, int32_t T, float rope_base, int32_t *dev_status,
                     void *stream) {
  if (!pos) return KVD_ERR_NULL;
  return append_impl(cache, k_new, v_new, 0, pos, dev_status, T, rope_base, stream);
}

int kv_reorder(const kvd_cache *cache, const int32_t *parent, int32_t len, int32_t *dev_status,
               void *stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (!parent) return KVD_ERR_NULL;
  if (len < 0 || cache->B > 16) return KVD_ERR_SHAPE;
  if (len > cache->S_max) return KVD_ERR_CAPACITY;
  if (!aligned4(parent) || (dev_status && !aligned4(dev_status))) return KVD_ERR_ALIGN;
  kvd::ReorderArgs a{};
  a.k_cache = cache->k;
  a.v_cache = cache->v;
  a.parent = parent;
  a.dev_status = dev_status;
  a.B = cache->B;
  a.H = cache->H;
  a.S_max = cache->S_max;
  a.len = len;
  return status_of(kvd::launch_reorder(cache->dtype, a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Shared by decode_attn_self and decode_step_self: validate and plan (no HIP
// call). k_new/v_new non-null: the N new rows are appended in the same launch.
// lens non-null: per-row lengths on the device (a ragged batch), with len
// their planned maximum.
int prepare_self(AttnArgs &a, const void *q, const void *k_new, const void *v_new, int32_t Hq,
                 int32_t N, const kvd_cache *cache, int32_t len, float scale, float rope_base,
                 float *out, void *ws, size_t ws_bytes, const int32_t *lens = nullptr,
                 int32_t *dev_status = nullptr, const kvd_cache *src = nullptr,
                 const int32_t *parent = nullptr) {
  int st = check_cache(cache);
  if (st) return st;
  if (!q || !out) return KVD_ERR_NULL;
  if (N < 1 || Hq < 1 || Hq % cache->H != 0 || !isfinite(scale) || !(rope_base >= 0.f) ||
      isinf(rope_base))
    return KVD_ERR_SHAPE;
  if (len > cache->S_max || len < N) return KVD_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(out)) return KVD_ERR_ALIGN;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return KVD_ERR_ALIGN;
  if ((lens && !aligned4(lens)) || (dev_status && !aligned4(dev_status))) return KVD_ERR_ALIGN;
  a = AttnArgs{};
  a.lens = lens;
  a.dev_status = dev_status;
  if (parent) {
    a.parent = parent;
    a.k_src = src->k;
    a.v_src = src->v;
  }
  a.q = q;
  a.k = cache->k;
  a.v = cache->v;
  a.k_new = k_new;
  a.v_new = v_new;
  a.out = out;
  a.B = cache->B;
  a.Hq = Hq;
  a.N = N;
  a.Bkv = cache->B;
  a.Hkv = cache->H;
  a.group = Hq / cache->H;
  a.S_max = cache->S_max;
  a.G = a.group * N;
  a.L = len;
  a.causal_base = len - N;
  a.new_base = k_new ? len - N : INT_MAX;
  a.T_new = k_new ? N : 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.rope_base = rope_base;
  a.rope_ratio = exp2(-(rope_base > 0.f ? 2.0 * log2((double)rope_base) / kvd::kHeadDim : 0.0));
  if (!rope_theta_of(rope_base, a.rope_theta)) return KVD_ERR_SHAPE;
  return prepare_attn(a, cache->dtype, ws, ws_bytes);
}

}  // namespace

int kvd::step_self(const void *q, const void *k_new, const void *v_new, int32_t Hq, int32_t N,
                   const kvd_cache *cache, int32_t len, float scale, float rope_base, float *out,
                   void *ws, size_t ws_bytes, void *stream, bool check_only) {
  if (!k_new || !v_new) return KVD_ERR_NULL;
  const bool fused = N <= kvd::kMaxFusedRows;
  AttnArgs a{};
  const int st = prepare_self(a, q, fused ? k_new : nullptr, fused ? v_new : nullptr, Hq, N, cache,
                              len, scale, rope_base, out, ws, ws_bytes);
  if (st) return st;
  if (!fused && (!aligned16(k_new) || !aligned16(v_new))) return KVD_ERR_ALIGN;
  if (check_only) return KVD_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!fused) {
    // a long block of new rows (prefill): append first, then attend
    kvd::AppendArgs ap{};
    ap.k_cache = cache->k;
    ap.v_cache = cache->v;
    ap.k_new = k_new;
    ap.v_new = v_new;
    ap.B = cache->B;
    ap.H = cache->H;
    ap.S_max = cache->S_max;
    ap.T = N;
    ap.pos = len - N;
    ap.rope_base = rope_base;
    ap.rope_theta = a.rope_theta;  // built (and checked) by prepare_self
    const int sa = status_of(kvd::launch_append(cache->dtype, ap, s));
    if (sa) return sa;
  }
  return status_of(kvd::launch_attn(cache->dtype, a, s));
}

extern "C" {

int decode_attn_self(const void *q, int32_t Hq, int32_t N, const kvd_cache *cache, int32_t len,
                     float scale, float rope_base, float *out, void *ws, size_t ws_bytes,
                     void *stream) {
  AttnArgs a{};
  const int st = prepare_self(a, q, nullptr, nullptr, Hq, N, cache, len, scale, rope_base, out,
                              ws, ws_bytes);
  if (st) return st;
  return status_of(kvd::launch_attn(cache->dtype, a, static_cast<hipStream_t>(stream)));
}

int decode_step_self(const void *q, const void *k_new, const void *v_new, int32_t Hq, int32_t N,
                     const kvd_cache *cache, int32_t len, float scale, float rope_base,
                     float *out, void *ws, size_t ws_bytes, void *stream) {
  return kvd::step_self(q, k_new, v_new, Hq, N, cache, len, scale, rope_base, out, ws, ws_bytes,
                        stream, false);
}

int decode_attn_self_ragged(const void *q, int32_t Hq, int32_t N, const kvd_cache *cache,
                            const int32_t *lens, int32_t len_max, float scale, float rope_base,
                            float *out, void *ws, size_t ws_bytes, int32_t *dev_status,
                            void *stream) {
  if (!lens) return KVD_ERR_NULL;
  AttnArgs a{};
  const int st = prepare_self(a, q, nullptr, nullptr, Hq, N, cache, len_max, scale, rope_base,
                              out, ws, ws_bytes, lens, dev_status);
  if (st) return st;
  return status_of(kvd::launch_attn(cache->dtype, a, static_cast<hipStream_t>(stream)));
}

int decode_step_self_ragged(const void *q, const void *k_new, const void *v_new, int32_t Hq,
                            int32_t N, const kvd_cache *cache, const int32_t *lens,
                            int32_t len_max, float scale, float rope_base, float *out, void *ws,
                            size_t ws_bytes, int32_t *dev_status, void *stream) {
  if (!k_new || !v_new || !lens) return KVD_ERR_NULL;
  if (N > kvd::kMaxFusedRows) return KVD_ERR_SHAPE;
  AttnArgs a{};
  const int st = prepare_self(a, q, k_new, v_new, Hq, N, cache, len_max, scale, rope_base, out,
                              ws, ws_bytes, lens, dev_status);
  if (st) return st;
  return status_of(kvd::launch_attn(cache->dtype, a, static_cast<hipStream_t>(stream)));
}

int decode_step_self_beams(const void *q, const void *k_new, const void *v_new, int32_t Hq,
                           int32_t N, const kvd_cache *src, const kvd_cache *dst,
                           const int32_t *parent, int32_t len, float scale, float rope_base,
                           float *out, void *ws, size_t ws_bytes, int32_t *dev_status,
                           void *stream) {
  int st = check_cache(src);
  if (st) return st;
  st = check_cache(dst);
  if (st) return st;
  if (!k_new || !v_new || !parent) return KVD_ERR_NULL;
  if (src->dtype != dst->dtype) return KVD_ERR_DTYPE;
  if (src->B != dst->B || src->H != dst->H || src->S_max != dst->S_max || N > kvd::kMaxFusedRows)
    return KVD_ERR_SHAPE;
  // beams read parents' rows of src while writing their own rows of dst:
  // the two caches' storage must not overlap
  const uintptr_t bytes = (uintptr_t)src->B * src->H * src->S_max * kvd::kHeadDim *
                          (src->dtype == KVD_F32 ? 4 : 2);
  const void *sp[2] = {src->k, src->v}, *dp[2] = {dst->k, dst->v};
  for (const void *x : sp)
    for (const void *y : dp) {
      const uintptr_t u = reinterpret_cast<uintptr_t>(x), w = reinterpret_cast<uintptr_t>(y);
      if (u < w + bytes && w < u + bytes) return KVD_ERR_SHAPE;
    }
  if (!aligned4(parent)) return KVD_ERR_ALIGN;
  AttnArgs a{};
  st = prepare_self(a, q, k_new, v_new, Hq, N, dst, len, scale, rope_base, out, ws, ws_bytes,
                    nullptr, dev_status, src, parent);
  if (st) return st;
  return status_of(kvd::launch_attn(dst->dtype, a, static_cast<hipStream_t>(stream)));
}

int decode_attn_cross(const void *q, int32_t B, int32_t Hq, int32_t N, const kvd_cache *xcache,
                      int32_t frames, float scale, float *out, void *ws, size_t ws_bytes,
                      void *stream) {
  int st = check_cache(xcache);
  if (st) return st;
  if (!q || !out) return KVD_ERR_NULL;
  if (B < 1 || N < 1 || Hq < 1 || Hq % xcache->H != 0 || !isfinite(scale) || frames < 1 ||
      (xcache->B != 1 && xcache->B != B))
    return KVD_ERR_SHAPE;
  if (frames > xcache->S_max) return KVD_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(out)) return KVD_ERR_ALIGN;
  AttnArgs a{};
  a.q = q;
  a.k = xcache->k;
  a.v = xcache->v;
  a.out = out;
  a.B = B;
  a.Hq = Hq;
  a.N = N;
  a.Bkv = xcache->B;
  a.Hkv = xcache->H;
  a.group = Hq / xcache->H;
  a.S_max = xcache->S_max;
  a.G = (xcache->B == 1 ? B : 1) * a.group * N;
  a.L = frames;
  a.causal_base = -1;
  a.new_base = INT_MAX;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.rope_base = 0.f;
  st = prepare_attn(a, xcache->dtype, ws, ws_bytes);
  if (st) return st;
  return status_of(kvd::launch_attn(xcache->dtype, a, static_cast<hipStream_t>(stream)));
}

size_t kvd_attn_workspace_bytes(int32_t B, int32_t Hq, int32_t N, int32_t len_max) {
  if (B < 1 || Hq < 1 || N < 1 || len_max < 1) return 0;
  // The largest plan over every grouping the calls can use (Hkv divides Hq,
  // cache per row or shared), every dtype, with and without rotary keys
  // (the plans differ: rotary ones keep 4 waves and split more) and every
  // length up to len_max.
  size_t best = 0;
  for (int hkv = 1; hkv <= Hq; ++hkv) {
    if (Hq % hkv) continue;
    const int group = Hq / hkv;
    for (int shared = 0; shared < 2; ++shared) {
      if (shared && B == 1) continue;
      const int units = shared ? hkv : B * hkv;
      const int G = (shared ? B : 1) * group * N;
      // fp32, 16-bit on matrix-core tiles, 16-bit streaming (the beam step)
      for (int dt = 0; dt < 3; ++dt) {
        for (int rope = 0; rope < 2; ++rope) {
          for (int L = 1; L <= len_max; ++L) {
            const AttnPlan p = kvd::plan_attn(dt == 0 ? kvd::F32 : kvd::F16, units, G, N, L,
                                              rope != 0, dt != 2);
            if (p.splits > 1) {
              const size_t b = attn_bytes(p);
              if (b > best) best = b;
            }
          }
        }
      }
    }
  }
  return best;
}

}  // extern "C"

namespace {

// verify_accept with optional suppression bitmaps; min_n is the smallest
// draft count the entry point accepts.
int verify_impl(const void *logits, int32_t logits_dtype, int32_t B, int32_t R, int32_t V,
                const int32_t *draft, int32_t N, int min_n, const uint32_t *suppress,
                const uint32_t *suppress_first, int32_t *argmax_out, int32_t *accept_len,
                int32_t *next_token, void *ws, size_t ws_bytes, void *stream) {
  if (!logits || (N > 0 && !draft) || !accept_len || !next_token) return KVD_ERR_NULL;
  if (!dtype_ok(logits_dtype)) return KVD_ERR_DTYPE;
  if (B < 1 || N < min_n || V < 1 || N > 63 || B > kvd::kMaxCounters) return KVD_ERR_SHAPE;
  if (R != N && R != N + 1) return KVD_ERR_ROWS;
  if (R < 1) return KVD_ERR_ROWS;
  int chunk = 0, chunks = 0;
  kvd::plan_verify(B, R, V, chunk, chunks);
  if (chunks > kvd::kMaxVerifyChunks) return KVD_ERR_SHAPE;
  if (!elem_aligned(logits, logits_dtype)) return KVD_ERR_ALIGN;
  if ((draft && !aligned4(draft)) || !aligned4(accept_len) || !aligned4(next_token) ||
      (argmax_out && !aligned4(argmax_out)) || (suppress && !aligned4(suppress)) ||
      (suppress_first && !aligned4(suppress_first)))
    return KVD_ERR_ALIGN;
  const size_t need = kvd_verify_workspace_bytes(B, R, V);
  if (!ws || ws_bytes < need) return KVD_ERR_WORKSPACE;
  if (!aligned16(ws)) return KVD_ERR_ALIGN;
  kvd::VerifyArgs a{};
  a.logits = logits;
  a.dtype = logits_dtype;
  a.draft = draft;
  a.argmax_out = argmax_out;
  a.accept_len = accept_len;
  a.next_token = next_token;
  a.suppress = suppress;
  a.suppress_first = suppress_first;
  a.B = B;
  a.R = R;
  a.V = V;
  a.N = N;
  a.chunk = chunk;
  a.chunks = chunks;
  a.ws_count = static_cast<uint32_t *>(ws);
  a.ws_key = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + kCounterBytes);
  return status_of(kvd::launch_verify(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int verify_accept(const void *logits, int32_t logits_dtype, int32_t B, int32_t R, int32_t V,
                  const int32_t *draft, int32_t N, int32_t *argmax_out, int32_t *accept_len,
                  int32_t *next_token, void *ws, size_t ws_bytes, void *stream) {
  if (!draft) return KVD_ERR_NULL;
  return verify_impl(logits, logits_dtype, B, R, V, draft, N, 1, nullptr, nullptr, argmax_out,
                     accept_len, next_token, ws, ws_bytes, stream);
}

int verify_accept_masked(const void *logits, int32_t logits_dtype, int32_t B, int32_t R,
                         int32_t V, const int32_t *draft, int32_t N, const uint32_t *suppress,
                         const uint32_t *suppress_first, int32_t *argmax_out,
                         int32_t *accept_len, int32_t *next_token, void *ws, size_t ws_bytes,
                         void *stream) {
  return verify_impl(logits, logits_dtype, B, R, V, draft, N, 0, suppress, suppress_first,
                     argmax_out, accept_len, next_token, ws, ws_bytes, stream);
}

size_t kvd_beam_workspace_bytes(int32_t B, int32_t K, int32_t V) {
  if (B < 1 || K < 1 || V < 1) return 0;
  return kCounterBytes + (size_t)B * K * kvd::beam_chunks(V) * kvd::kBeamRec * sizeof(uint32_t);
}

int beam_select(const void *logits, int32_t logits_dtype, int32_t B, int32_t K, int32_t V,
                const float *sum_logprobs, int32_t eot, int32_t *parent, int32_t *token,
                float *score, int32_t *finished_count, int32_t *finished_parent,
                float *finished_score, void *ws, size_t ws_bytes, void *stream) {
  if (!logits || !sum_logprobs || !parent || !token || !score || !finished_count ||
      !finished_parent || !finished_score)
    return KVD_ERR_NULL;
  if (!dtype_ok(logits_dtype)) return KVD_ERR_DTYPE;
  if (B < 1 || B > kvd::kMaxCounters || K < 1 || K > kvd::kMaxBeamWidth || V < K + 1)
    return KVD_ERR_SHAPE;
  const int chunks = kvd::beam_chunks(V);
  if ((int64_t)(K + 1) * chunks > kvd::kMaxBeamEntries) return KVD_ERR_SHAPE;
  if (!elem_aligned(logits, logits_dtype) || !aligned4(sum_logprobs) || !aligned4(parent) ||
      !aligned4(token) ||
      !aligned4(score) || !aligned4(finished_count) || !aligned4(finished_parent) ||
      !aligned4(finished_score))
    return KVD_ERR_ALIGN;
  if (!ws || ws_bytes < kvd_beam_workspace_bytes(B, K, V)) return KVD_ERR_WORKSPACE;
  if (!aligned16(ws)) return KVD_ERR_ALIGN;
  kvd::BeamArgs a{};
  a.logits = logits;
  a.dtype = logits_dtype;
  a.sum_logprobs = sum_logprobs;
  a.parent = parent;
  a.token = token;
  a.score = score;
  a.fin_count = finished_count;
  a.fin_parent = finished_parent;
  a.fin_score = finished_score;
  a.ws_count = static_cast<uint32_t *>(ws);
  a.ws_rec = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + kCounterBytes);
  a.B = B;
  a.K = K;
  a.V = V;
  a.eot = eot;
  a.chunks = chunks;
  return status_of(kvd::launch_beam(a, static_cast<hipStream_t>(stream)));
}

size_t kvd_verify_workspace_bytes(int32_t B, int32_t R, int32_t V) {
  if (B < 1 || R < 1 || V < 1) return 0;
  int chunk = 0, chunks = 0;
  kvd::plan_verify(B, R, V, chunk, chunks);
  return kCounterBytes + (size_t)B * R * chunks * sizeof(uint64_t);
}

}  // extern "C"
