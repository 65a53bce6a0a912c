/*
 * kvdecode.h - C ABI of the KV-cached decoder-step library for AMD MI355X
 * (gfx950). Plain C types only; every pointer named "device" is HIP device
 * memory, every other pointer is host memory.
 *
 * Sources the operations follow (page title, section):
 *   [W] "Whisper のデコーダー内部：Beam Search、Logit フィルター、KV キャッシュ"
 *       (readoss.com): section "Inference 抽象と KV キャッシュ" - the
 *       save_to_cache hook (self-attention K/V concatenated onto the cache,
 *       cross-attention K/V stored once from the encoder output and reused),
 *       the greedy decoder (argmax at temperature 0) and step 4 of the beam
 *       search update (reorder the cache to the new beam order).
 *   [N] "nanoVLM における KV キャッシュ実装" (agentlenshq.com): sections
 *       "KV キャッシュが推論を最適化する方法" (per-layer key/value tensors of
 *       shape (batch, heads, seq_cached, head_dim); new K/V appended, then the
 *       current query attends over the cache) and "nanoVLM における技術的実装"
 *       (grouped-query attention; start_pos keeps rotary positions absolute;
 *       prefill then decode).
 *   [S] "추측 디코딩으로 Whisper 추론 속도 2배 향상" (agentlenshq.com), section
 *       "추측 디코딩이란?", and the aitime.ge translation of the same post
 *       (its worked example): the main model scores the drafts in one pass,
 *       drafts are kept up to the first mismatch, the main model's token
 *       replaces the mismatch and the rest is dropped.
 *
 * Conventions shared by every call
 *   - Element types: KVD_F32, KVD_F16 (IEEE binary16), KVD_BF16. Attention
 *     accumulates in fp32 and writes fp32 output.
 *   - Head dimension D must be 64.
 *   - All device buffers are contiguous, row-major in the order written, and
 *     16-byte aligned, except where a call states otherwise. The caller owns
 *     every buffer; the library allocates nothing and keeps no state between
 *     calls (besides the testing hook's forced plan).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream). Calls are thread-safe; two calls that share a
 *     workspace must be ordered (same stream).
 *   - Return value: KVD_OK, or a negative status. Every status except
 *     KVD_ERR_LAUNCH is decided on the host before any HIP call, so nothing is
 *     enqueued when a call fails.
 *   - Results are deterministic: split counts depend only on the shape and
 *     every reduction runs in a fixed order. The one exception is a plan a
 *     test forces with kvd_set_plan_override (declared below, off unless
 *     called); the library reads no environment variable.
 */
#ifndef KVDECODE_H
#define KVDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kvd_dtype { KVD_F32 = 0, KVD_F16 = 1, KVD_BF16 = 2 };

enum kvd_status {
  KVD_OK = 0,
  KVD_ERR_NULL = -1,       /* a required pointer is NULL */
  KVD_ERR_SHAPE = -2,      /* a size is out of range or two sizes disagree */
  KVD_ERR_DTYPE = -3,      /* unknown element type */
  KVD_ERR_CAPACITY = -4,   /* rows beyond the cache capacity S_max */
  KVD_ERR_ROWS = -5,       /* verify: logits rows R is neither N nor N + 1 */
  KVD_ERR_WORKSPACE = -6,  /* workspace NULL or smaller than required */
  KVD_ERR_ALIGN = -7,      /* a device pointer is not 16-byte aligned */
  KVD_ERR_LAUNCH = -8,     /* the HIP launch reported an error */
  KVD_ERR_SCRATCH = -9     /* decode_step_self_static: the shape needs more
                              scratch than the library's static array holds */
};

/* One layer's K/V cache ([N] per-layer key/value tensors).
 * k, v: device, [B][H][S_max][D] elements of `dtype`. Rows [0, len) of every
 * (b, h) are valid; the library never reads past the `len` it is given. */
typedef struct kvd_cache {
  void *k;
  void *v;
  int32_t B;      /* batch rows (beams count as rows); 1 for a shared cross cache */
  int32_t H;      /* K/V heads */
  int32_t S_max;  /* capacity in positions */
  int32_t D;      /* head dimension (64) */
  int32_t dtype;  /* enum kvd_dtype */
} kvd_cache;

/* kv_append - write T new K/V rows per (b, h) at positions [pos, pos + T).
 * [W] save_to_cache (self attention: concatenation along the sequence;
 * cross attention: the encoder-derived K/V written once, here T = frames at
 * pos = 0); [N] workflow steps 2-3 and the prefill phase (T = prompt length).
 *   k_new, v_new: device, [B][H][T][D] in cache->dtype.
 *   rope_base > 0: each key row is first rotated at its absolute position
 *     pos + t (pairs (i, i + D/2) turn by (pos + t) * rope_base^(-2i/D));
 *     the angle is formed and reduced modulo pi/2 in fp64, its cos / sin
 *     (fp32 polynomials, error below 2^-23) and the rotation are computed in
 *     fp32, and the result is rounded to nearest-even into the cache; values
 *     are copied as they are.
 *     rope_base == 0: a bit-exact copy of both.
 * Errors: KVD_ERR_NULL, KVD_ERR_SHAPE (T < 1, pos < 0, D != 64, B/H < 1),
 *   KVD_ERR_DTYPE, KVD_ERR_CAPACITY (pos + T > S_max), KVD_ERR_ALIGN. */
int kv_append(const kvd_cache *cache, const void *k_new, const void *v_new,
              int32_t pos, int32_t T, float rope_base, void *stream);

/* kv_reorder - beam reorder in place: rows [0, len) of beam b, K and V of
 * every head, become the rows beam parent[b] held before the call.
 * [W] beam search update, step 4 (rearrange_kv_cache).
 *   parent: device int32[cache->B]; repeats allowed (several beams may take
 *     the same parent); parent[b] == b leaves beam b untouched.
 *   dev_status: device int32 or NULL. A parent outside [0, B) leaves that
 *     beam unchanged and stores KVD_ERR_SHAPE there (never faults).
 * Errors: KVD_ERR_NULL, KVD_ERR_SHAPE (len < 0, B > 16, D != 64),
 *   KVD_ERR_DTYPE, KVD_ERR_CAPACITY (len > S_max), KVD_ERR_ALIGN. */
int kv_reorder(const kvd_cache *cache, const int32_t *parent, int32_t len,
               int32_t *dev_status, void *stream);

/* decode_attn_self - attention of N new queries over a self-attention cache
 * that already holds them ([W]: attention sees the whole concatenated
 * sequence; [N] workflow step 4; [S]: the N drafts scored in one pass).
 *   q: device, [B][Hq][N][D] in cache->dtype, B = cache->B. Query i sits at
 *     position len - N + i and sees keys 0 .. len - N + i (causal among the
 *     N new rows). Query head h reads K/V head h / (Hq / cache->H).
 *   len: valid cache rows after the append, N <= len <= S_max.
 *   scale: multiplies q.k (1/sqrt(D) for the usual attention).
 *   rope_base > 0: query i is rotated at position len - N + i first (same
 *     rotation as kv_append); 0: no rotation.
 *   out: device fp32 [B][Hq][N][D] = softmax(scale q K^T) V.
 *   ws: device workspace of ws_bytes >= kvd_attn_workspace_bytes(B, Hq, N,
 *     len); it must be zero-filled before its first use and is left that way.
 * Errors: KVD_ERR_NULL, KVD_ERR_SHAPE (N < 1, Hq % H != 0, D != 64),
 *   KVD_ERR_DTYPE, KVD_ERR_CAPACITY (len > S_max or len < N),
 *   KVD_ERR_WORKSPACE, KVD_ERR_ALIGN. */
int decode_attn_self(const void *q, int32_t Hq, int32_t N, const kvd_cache *cache,
                     int32_t len, float scale, float rope_base, float *out,
                     void *ws, size_t ws_bytes, void *stream);

/* decode_step_self - kv_append followed by decode_attn_self, in one launch
 * for N <= 16 (two launches on `stream` for longer blocks such as a prefill):
 * the N new K/V rows are written at positions [len - N, len) (keys rotated
 * exactly as kv_append rotates them when rope_base > 0) and the N queries
 * attend over the cache including them ([W] the hook returns the cache with
 * the new rows concatenated, and attention consumes that; [N] attention
 * block: concatenate K_new/V_new onto the cache, then attend).
 *   k_new, v_new: device, [B][H][N][D] in cache->dtype (B, H of the cache).
 *   Other arguments, results and errors as decode_attn_self. After the call
 *   the cache holds exactly what kv_append(cache, k_new, v_new, len - N, N,
 *   rope_base) would have written, and `out` equals what decode_attn_self
 *   would have returned. */
int decode_step_self(const void *q, const void *k_new, const void *v_new, int32_t Hq, int32_t N,
                     const kvd_cache *cache, int32_t len, float scale, float rope_base,
                     float *out, void *ws, size_t ws_bytes, void *stream);

/* Ragged batches ([S] applied to a batch of sequences: each batch row
 * accepts its own number of drafts, so its cache length moves on its own).
 * The calls below take per-row positions or lengths in a device array, so a
 * decode loop never reads them back to the host; a rolled-back row simply
 * gets a shorter length (rows past it are overwritten later).
 *
 * kv_append_ragged - kv_append with row b written at [pos[b], pos[b] + T).
 *   pos: device int32 [cache->B]. A row whose pos[b] < 0 or
 *     pos[b] + T > S_max is not written and KVD_ERR_CAPACITY is stored in
 *     dev_status (device int32, or NULL); other rows are written.
 *   Other arguments and errors as kv_append. */
int kv_append_ragged(const kvd_cache *cache, const void *k_new, const void *v_new,
                     const int32_t *pos, int32_t T, float rope_base, int32_t *dev_status,
                     void *stream);

/* decode_attn_self_ragged - decode_attn_self with row b's length lens[b]:
 * its query i sits at position lens[b] - N + i and sees keys
 * 0 .. lens[b] - N + i.
 *   lens: device int32 [cache->B]; len_max: a host bound, N <= len_max <=
 *     S_max, that the split plan and the workspace are sized for
 *     (kvd_attn_workspace_bytes(B, Hq, N, len_max)). A lens[b] outside
 *     [N, len_max] is clamped into it and KVD_ERR_CAPACITY is stored in
 *     dev_status (device int32, or NULL).
 *   Other arguments, results and errors as decode_attn_self with
 *   len = len_max. */
int decode_attn_self_ragged(const void *q, int32_t Hq, int32_t N, const kvd_cache *cache,
                            const int32_t *lens, int32_t len_max, float scale, float rope_base,
                            float *out, void *ws, size_t ws_bytes, int32_t *dev_status,
                            void *stream);

/* decode_step_self_static - decode_step_self for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): no workspace argument; the split merge
 * uses a static device array of kvd_static_scratch_bytes() (4 MiB) that
 * each GPU holds until the process ends. The call itself allocates nothing.
 *   Arguments, results and bits of `out` as decode_step_self.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (several streams or threads at once) race and must be ordered by the
 *   caller. The first call on a GPU clears the array's counter block with a
 *   kernel on `stream` (inside a stream capture, once per captured graph).
 * Errors: as decode_step_self, KVD_ERR_SCRATCH when the shape's merge needs
 *   more than the array holds (it holds every Whisper-large-v2 and 8-row GQA
 *   decode step; kvd_attn_workspace_bytes(B, Hq, N, len) <= 4 MiB), and
 *   KVD_ERR_LAUNCH if the device array cannot be found. */
int decode_step_self_static(const void *q, const void *k_new, const void *v_new, int32_t Hq,
                            int32_t N, const kvd_cache *cache, int32_t len, float scale,
                            float rope_base, float *out, void *stream);
size_t kvd_static_scratch_bytes(void);

/* decode_step_self_ragged - decode_step_self with per-row lengths, in one
 * launch (N <= 16): row b's N new K/V rows are written at
 * [lens[b] - N, lens[b]) and its queries attend as in
 * decode_attn_self_ragged. After the call the cache holds exactly what
 * kv_append_ragged at positions lens[b] - N would have written.
 * Errors as decode_attn_self_ragged, and KVD_ERR_SHAPE for N > 16. */
int decode_step_self_ragged(const void *q, const void *k_new, const void *v_new, int32_t Hq,
                            int32_t N, const kvd_cache *cache, const int32_t *lens,
                            int32_t len_max, float scale, float rope_base, float *out, void *ws,
                            size_t ws_bytes, int32_t *dev_status, void *stream);

/* decode_step_self_beams - one beam-search decode step on two caches used in
 * turn: kv_reorder, then decode_step_self, in one launch (N <= 16), with the
 * reordered rows written into a second cache instead of in place ([W] beam
 * search update, step 4, rearrange_kv_cache, followed by the next step's
 * append and attention). For every beam b, rows [0, len - N) of every head
 * of dst become rows [0, len - N) of beam parent[b] in src; the N new K/V
 * rows go to [len - N, len) of dst; the queries attend over dst as
 * decode_step_self does. Each cached row is read once, for both the copy and
 * the attention. The caller swaps src and dst for the next step.
 *   src, dst: caches of equal dtype, B, H and S_max whose storage does not
 *     overlap (src is only read); rows of dst from len on are not touched.
 *   parent: device int32 [B], repeats allowed. A parent outside [0, B)
 *     makes beam b read its own rows of src and stores KVD_ERR_SHAPE in
 *     dev_status (device int32, or NULL).
 *   ws: kvd_attn_workspace_bytes(B, Hq, N, len).
 *   Other arguments and results as decode_step_self on dst. After the call
 *   dst holds exactly what the copy and kv_append(dst, k_new, v_new, len - N,
 *   N, rope_base) would have written, and `out` equals decode_attn_self's.
 * Errors: as decode_step_self; KVD_ERR_DTYPE when the dtypes differ;
 *   KVD_ERR_SHAPE when B, H or S_max differ, the storage overlaps, or
 *   N > 16. */
int decode_step_self_beams(const void *q, const void *k_new, const void *v_new, int32_t Hq,
                           int32_t N, const kvd_cache *src, const kvd_cache *dst,
                           const int32_t *parent, int32_t len, float scale, float rope_base,
                           float *out, void *ws, size_t ws_bytes, int32_t *dev_status,
                           void *stream);

/* decode_attn_cross - attention of N queries per row over all `frames`
 * rows of a cross-attention cache, with no mask ([W]: cross-attention K/V
 * computed once from the encoder and reused every step).
 *   q: device, [B][Hq][N][D] in xcache->dtype.
 *   xcache->B == 1: one cache shared by all B rows (beams of one audio);
 *     xcache->B == B: one cache per row.
 *   frames: 1 <= frames <= xcache->S_max.
 *   out: device fp32 [B][Hq][N][D]; ws as for decode_attn_self
 *     (kvd_attn_workspace_bytes(B, Hq, N, frames)).
 * Errors: as decode_attn_self; KVD_ERR_SHAPE also when xcache->B is
 *   neither 1 nor B. */
int decode_attn_cross(const void *q, int32_t B, int32_t Hq, int32_t N,
                      const kvd_cache *xcache, int32_t frames, float scale,
                      float *out, void *ws, size_t ws_bytes, void *stream);

/* verify_accept - speculative verification epilogue ([S]; [W] greedy
 * argmax). For each batch row b:
 *   argmax[r] = lowest index of the largest logit of row r (-inf is an
 *     ordinary value; a row of only -inf gives 0; NaN is outside the
 *     contract),
 *   accept_len[b] = n = first i < N with draft[b][i] != argmax[i], else N,
 *   next_token[b] = argmax[n] if n < R, else -1 (all N drafts kept and no
 *     bonus row).
 *   logits: device, [B][R][V] of logits_dtype, aligned to its element; R = N
 *     (row i scores draft i)
 *     or N + 1 (a bonus row after the last draft).
 *   draft: device int32 [B][N] (any value; one outside [0, V) never matches).
 *   argmax_out: device int32 [B][R] or NULL.
 *   accept_len, next_token: device int32 [B].
 *   ws: device workspace, ws_bytes >= kvd_verify_workspace_bytes(B, R, V),
 *     zero-filled before its first use and left that way.
 * Errors: KVD_ERR_NULL, KVD_ERR_SHAPE (B, N, V < 1; N > 63; B > 4096;
 *   V > 1048576), KVD_ERR_ROWS,
 *   KVD_ERR_DTYPE, KVD_ERR_WORKSPACE, KVD_ERR_ALIGN (logits not aligned to
 *   their element, other pointers to 4 bytes). */
int verify_accept(const void *logits, int32_t logits_dtype, int32_t B, int32_t R,
                  int32_t V, const int32_t *draft, int32_t N, int32_t *argmax_out,
                  int32_t *accept_len, int32_t *next_token, void *ws,
                  size_t ws_bytes, void *stream);

/* verify_accept_masked - verify_accept after the logit filters of [W]
 * (section "LogitFilter チェーン": SuppressTokens sets a fixed token list to
 * -inf on every step, SuppressBlank sets the blank and end-of-text tokens to
 * -inf at the first sampled position; section "言語検出": every token but the
 * language tokens at -inf, then argmax). A suppressed logit counts as -inf
 * and the argmax then follows verify_accept's rules.
 *   suppress: device bitmap of ceil(V / 32) uint32 words (bit t % 32 of word
 *     t / 32 set: token t suppressed) applied to every row, or NULL.
 *   suppress_first: the same, applied in addition to row 0 of each batch row
 *     (the first sampled position), or NULL.
 *   N may be 0 (draft may then be NULL) with R = 1: next_token[b] is the
 *     filtered argmax of the one row, as in a greedy step or language
 *     detection.
 *   Other arguments, the workspace (kvd_verify_workspace_bytes(B, R, V)) and
 *   the errors are those of verify_accept; the bitmaps must be 4-byte
 *   aligned. */
int verify_accept_masked(const void *logits, int32_t logits_dtype, int32_t B, int32_t R,
                         int32_t V, const int32_t *draft, int32_t N, const uint32_t *suppress,
                         const uint32_t *suppress_first, int32_t *argmax_out,
                         int32_t *accept_len, int32_t *next_token, void *ws, size_t ws_bytes,
                         void *stream);

/* beam_select - one beam-search update for each audio row b, following the
 * beam-search decoder's update steps on [W] (step 4, reordering the caches
 * to the new beam order, is kv_reorder with the `parent` produced here):
 *   1. log-probabilities of each beam's logits row (natural-log softmax) and
 *      the beam's K + 1 best tokens (larger logit first; equal logits: lower
 *      token first);
 *   2. candidate (beam j, token t) scores sum_logprobs[b][j] + logp_j(t);
 *   3. candidates are taken in order of score (larger first; equal scores
 *      in the order beam, then rank): an `eot` token is recorded as finished,
 *      any other token becomes the next beam, until K next beams are chosen.
 *   logits: device, [B][K][V] of logits_dtype, aligned to its element; every
 *     row needs a finite maximum (NaN is outside the contract).
 *   sum_logprobs: device fp32 [B][K], the beams' running scores.
 *   eot: end-of-text token (any value; one outside [0, V) never matches).
 *   parent, token: device int32 [B][K]: next beam k continues beam
 *     parent[b][k] with token[b][k]; score: device fp32 [B][K], its running
 *     score (log-probabilities and scores in fp32).
 *   finished_count: device int32 [B]; finished_parent (int32) and
 *     finished_score (fp32): device [B][K], the first finished_count entries
 *     in the order met, then -1 / NaN.
 *   ws: device workspace of ws_bytes >= kvd_beam_workspace_bytes(B, K, V),
 *     zero-filled before its first use and left that way.
 * Errors: KVD_ERR_NULL, KVD_ERR_DTYPE, KVD_ERR_SHAPE (B < 1, B > 4096,
 *   K outside [1, 16], V < K + 1, (K + 1) * ceil(V / 2048) > 512: e.g.
 *   V <= 61440 at K = 16, V <= 174080 at K = 5),
 *   KVD_ERR_WORKSPACE, KVD_ERR_ALIGN. */
int beam_select(const void *logits, int32_t logits_dtype, int32_t B, int32_t K, int32_t V,
                const float *sum_logprobs, int32_t eot, int32_t *parent, int32_t *token,
                float *score, int32_t *finished_count, int32_t *finished_parent,
                float *finished_score, void *ws, size_t ws_bytes, void *stream);

/* Workspace sizes (bytes) for the calls above: 0 for invalid sizes, and 0
 * when no call of that shape merges split partials (a NULL workspace is then
 * accepted). A workspace sized for the largest len (or frames) serves every
 * smaller one. */
size_t kvd_attn_workspace_bytes(int32_t B, int32_t Hq, int32_t N, int32_t len_max);
size_t kvd_verify_workspace_bytes(int32_t B, int32_t R, int32_t V);
size_t kvd_beam_workspace_bytes(int32_t B, int32_t K, int32_t V);

/* Measurement aid: a plain streaming read of `bytes` from a and, when b is
 * not NULL, `bytes` from b, in one launch on `stream` (every 16-byte vector
 * is loaded once; nothing is written except, with negligible probability, one
 * word at `sink`). Its duration is the attainable time for a kernel that
 * reads that many bytes once, the yardstick for the attention kernels.
 *   a, b: device, 16-byte aligned; bytes: a multiple of 16, > 0.
 *   sink: device uint32, 4-byte aligned.
 * Errors: KVD_ERR_NULL, KVD_ERR_SHAPE, KVD_ERR_ALIGN, KVD_ERR_LAUNCH. */
int kvd_read_probe(const void *a, const void *b, size_t bytes, uint32_t *sink, void *stream);

/* The same read with its shape chosen by the caller, so that the yardstick
 * can be the fastest of several: every thread keeps `unroll` 16-byte loads in
 * flight per round (1, 2, 4, 8 or 16), over `blocks` workgroups of 256
 * threads (1 .. 65535; 0: enough for one round of loads per thread), reading
 * a's vectors and then b's as one grid-stride sequence. kvd_read_probe is
 * unroll 4, blocks 0.
 * Errors: as kvd_read_probe; KVD_ERR_SHAPE also for another unroll or
 * blocks > 65535. */
int kvd_read_probe_ex(const void *a, const void *b, size_t bytes, uint32_t *sink, int32_t unroll,
                      size_t blocks, void *stream);

/* Testing hook: force the split plan of every later attention call and
 * workspace query in this process, so tests can reach plans the shapes they
 * use would not get. mfma: -1 plan as usual, 0 keep 16-bit caches on the
 * streaming kernel (1 is the same as -1); waves: waves per workgroup (0: as
 * planned; the planner keeps only values its kernel supports); chunk: keys
 * per split (0: as planned). kvd_set_plan_override(-1, 0, 0) restores the
 * default, under which the plan is a pure function of the call's shape. A
 * workspace sized under one setting may be too small under another (the
 * call then returns KVD_ERR_WORKSPACE). Not for use while other threads
 * make calls.
 * Errors: KVD_ERR_SHAPE for values outside those ranges. */
int kvd_set_plan_override(int32_t mfma, int32_t waves, int32_t chunk);

/* Profiling aid: the next kernel launch made by the calling thread records
 * `start_event` when the kernel begins and `stop_event` when it ends (created
 * hipEvent_t handles, or NULL), so hipEventElapsedTime gives the kernel's own
 * duration without launch gaps. The request is consumed by that one launch. */
int kvd_time_next_launch(void *start_event, void *stop_event);

/* Static text for a status code (never NULL). */
const char *kvd_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVDECODE_H */
