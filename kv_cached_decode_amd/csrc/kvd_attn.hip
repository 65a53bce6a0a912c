// Decode attention on gfx950, split over keys (the streaming kernel used for
// one query per head and for small query groups).
//
// Workgroup (split, row tile, unit) takes keys [split*chunk, +chunk) of one
// (cache row, kv head) "unit" for up to GM query rows. A wavefront loads
// TILE keys per iteration with 16-byte loads: LPR lanes share a key row, so
// one wave load covers RPL whole rows and is fully coalesced. Scores are
// reduced across the LPR lanes with DPP. Each group of LPR lanes keeps its
// own online-softmax state (running max m, sum l, unnormalised o, in the log2
// domain), so the key loop has no cross-group traffic; groups are merged once
// per wave, waves once per workgroup in LDS. Splits are merged by the last
// workgroup of the tile to arrive, in split order, so the result does not
// depend on arrival order.
//
// With new rows (k_new/v_new, at most kMaxFusedRows of them), the kernel also
// performs the cache append of the step: each workgroup rotates and rounds
// the new rows of its key range once into LDS, exactly as kv_append would
// store them, and reads them from there; the workgroups of row tile 0 write
// them into the cache. No workgroup reads those cache rows, so the writes
// need no ordering within the launch.
#include <stdlib.h>

#include <atomic>

#include "kvd_attn_common.hpp"
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

namespace {

constexpr int kSteps = 4;
template <int DT>
struct AttnGeom {
  static constexpr int VE = vec_elems<DT>();      // elements per lane load
  static constexpr int LPR = kHeadDim / VE;       // lanes per key row
  static constexpr int RPL = 64 / LPR;            // key rows per wave load
  static constexpr int TILE = RPL * kSteps;       // keys per wave iteration
  static constexpr int ROWB = kHeadDim * Storage<DT>::bytes;
};

template <int DT, int GM, bool FUSED, int NWMAX, bool ROPE, bool RAGGED, bool BEAM>
__global__ __launch_bounds__(64 * NWMAX) void attn_kernel(KVD_LEAD_PARAMS, AttnArgs args) {
  using Geo = AttnGeom<DT>;
  constexpr int D = kHeadDim;
  constexpr int VE = Geo::VE, LPR = Geo::LPR, RPL = Geo::RPL, TILE = Geo::TILE;
  constexpr int ROWB = Geo::ROWB;
  constexpr int VPR = ROWB / 16;  // 16-byte vectors per row
  // The struct: read through lead_struct() once the first key loads are out
  // (16-bit caches with no per-row lengths or beam parents, which the first
  // loads would need); otherwise the parameter itself, whose fields the
  // compiler fetches where they are used, and the lead values taken from it
  // too (fp32 kernels, which use more registers, would spill with both sets
  // held in scalar registers).
  constexpr bool kLateArgs = DT != F32 && !RAGGED && !BEAM;
  const Lead ld = kLateArgs ? KVD_LEAD
                            : Lead{static_cast<char *>(args.k), static_cast<char *>(args.v),
                                   FastDiv{lead_hkv_m, lead_hkv_s}, args.Hkv, args.S_max, args.chunk,
                                   args.L, args.causal_base, args.new_base, lead_nw};
  AttnArgs a;
  if constexpr (!kLateArgs) a = args;

  const int lane = threadIdx.x & 63;
  // wave-uniform values kept in scalar registers, so that the key loop and
  // its tests are scalar branches and not per-lane masks
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = ld.nw;
  const int kr = lane / LPR;  // key row within a wave load
  const int ds = lane % LPR;  // dims [ds*VE, ds*VE + VE)

  // ---- the unit, its key range and its rows' bases: preloaded arguments
  // only, so the first tiles' loads below wait for no memory access
  const int split = blockIdx.x, rt = blockIdx.y, unit = blockIdx.z;
  const int bkv = (int)fast_div((uint32_t)unit, ld.div_Hkv), hk = unit - bkv * ld.Hkv;
  const int k0 = split * ld.chunk;
  const RowSpan sp = row_span<RAGGED>(a, bkv, ld.L, ld.causal_base, ld.new_base);
  const int kspan = min(k0 + ld.chunk, sp.L);

  const size_t head = (size_t)unit;  // bkv * Hkv + hk: no division in front of the first loads
  char *kc = ld.k + head * ld.S_max * ROWB;
  char *vc = ld.v + head * ld.S_max * ROWB;
  const int nb0 = max(k0, sp.new_base);  // first new row of this key range
  // Where the cached rows are read: this unit's own rows, or (beam step:
  // reorder + append + attend) the rows of beam parent[b] in the source
  // cache, which row tile 0 also writes into this beam's rows of k / v.
  const char *ks = kc, *vs = vc;
  static_assert(!BEAM || FUSED, "the beam step appends its new rows");
  if constexpr (BEAM) {
    int p = a.parent[bkv];
    if (p < 0 || p >= a.Bkv) {  // outside the contract: keep this beam's own rows
      if (a.dev_status && threadIdx.x == 0) *a.dev_status = kStatusBadShape;
      p = bkv;
    }
    const size_t src = ((size_t)p * ld.Hkv + hk) * ld.S_max * ROWB;
    ks = static_cast<const char *>(a.k_src) + src;
    vs = static_cast<const char *>(a.v_src) + src;
  }

  // ---- first tiles: when every query row sees all keys of a tile (a causal
  // row sees at least keys 0 .. causal_base) and none of them is new, the
  // tile's loads go out first, before the query rows and the rows'
  // bookkeeping below. Without new rows, with few query rows and 4 waves
  // (registers to spare; measured to pay only there), each wave keeps two
  // tiles in flight: tile i + 2 is loaded into the buffer tile i just freed.
  constexpr int PF = (!FUSED && GM <= 2 && NWMAX <= 4) ? 2 : 1;
  // Fused steps without rotation or beam parents: the wave whose tile holds
  // new rows loads them straight from k_new / v_new into the tile's
  // registers (no LDS staging, no barrier) and row tile 0 writes them into
  // the cache from there. Otherwise they are staged through LDS.
  constexpr bool kRegNew = FUSED && !ROPE && !BEAM;
  u32x4 kA[kSteps], vA[kSteps], kB[PF == 2 ? kSteps : 1], vB[PF == 2 ? kSteps : 1];
  const int stride = nw * TILE;
  int t0 = k0 + wave * TILE;
  const int kend_lo = min(kspan, (sp.causal_base < 0) ? sp.L : sp.causal_base + 1);
  auto seen_by_all = [&](int t) { return t + TILE <= kend_lo && (!FUSED || t + TILE <= nb0); };
  auto load_plain = [&](u32x4 *kd, u32x4 *vd, int t) {  // a whole tile
    const char *kb = ks + (size_t)t * ROWB;
    const char *vb = vs + (size_t)t * ROWB;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const uint32_t off = (uint32_t)((s * RPL + kr) * ROWB + ds * 16);
      kd[s] = load16(kb + off);
      vd[s] = load16(vb + off);
    }
  };
  const bool early_a = seen_by_all(t0);                      // uniform
  const bool early_b = PF == 2 && seen_by_all(t0 + stride);  // uniform
  if (early_a) load_plain(kA, vA, t0);
  if constexpr (PF == 2) {
    if (early_b) load_plain(kB, vB, t0 + stride);
  }

  // ---- query rows (their numbering and q's base come from the struct);
  // vector loads complete in issue order, so they land after the first tiles
  if constexpr (kLateArgs) {
    a = lead_struct();
    // the fields the query rows' numbering and addresses (and the new rows'
    // loads) need, fetched in one round trip: left to the compiler, each
    // went out at its first use, three scalar round trips before the query
    // load
    asm volatile("" ::"s"(a.q), "s"(a.G), "s"(a.N), "s"(a.group), "s"(a.Hq), "s"(a.Bkv),
                 "s"(a.div_N.m), "s"(a.div_N.s), "s"(a.div_group.m), "s"(a.div_group.s));
    if constexpr (FUSED) asm volatile("" ::"s"(a.k_new), "s"(a.v_new), "s"(a.T_new));
  }
  const int g0 = rt * GM;
  const int gcount = min(GM, a.G - g0);
  u32x4 qraw[GM], qpart[GM];
  size_t orow[GM];  // element offset of each row in q's layout, which out shares
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    qraw[g] = u32x4{0, 0, 0, 0};
    qpart[g] = u32x4{0, 0, 0, 0};
    orow[g] = 0;
    if (g < gcount) {
      orow[g] = out_row(a, row_id(a, bkv, hk, g0 + g));
      const char *qrow = static_cast<const char *>(a.q) + orow[g] * Storage<DT>::bytes;
      qraw[g] = load16(qrow + ds * 16);
      if (ROPE) qpart[g] = load16(qrow + (ds ^ (LPR / 2)) * 16);
    }
  }

  // ---- which keys each query row sees (indices only, no memory access)
  int lim[GM];
  int kvis = 0;
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    lim[g] = 0;
    if (g < gcount) {
      const RowId r = row_id(a, bkv, hk, g0 + g);
      lim[g] = (sp.causal_base < 0) ? sp.L : sp.causal_base + r.i + 1;
      kvis = max(kvis, lim[g]);
    }
  }
  const int kend = __builtin_amdgcn_readfirstlane(min(kspan, kvis));

  // A whole tile of cached keys: plain loads from a uniform base plus 32-bit
  // lane offsets. A tile reaching past kend or into the new rows loads its
  // keys clamped to the last cached one (row 0 if there is none), again with
  // no branch and no zeroed register in front of a load (either would cost
  // instructions and make the compiler wait for earlier loads). Past kend the
  // scores are masked; the values there are rows below kend, so finite,
  // except with new rows (see the fused loop).
  const int kcap = max((FUSED ? min(kend, nb0) : kend) - 1, 0);
  auto whole = [&](int t) { return t + TILE <= kend && (!FUSED || t + TILE <= nb0); };
  // new rows of a tile, in registers of their own (kRegNew)
  u32x4 nk[kRegNew ? kSteps : 1], nv[kRegNew ? kSteps : 1];
  const char *knb = nullptr, *vnb = nullptr;
  if constexpr (kRegNew) {
    knb = static_cast<const char *>(a.k_new) + head * a.T_new * ROWB;
    vnb = static_cast<const char *>(a.v_new) + head * a.T_new * ROWB;
  }
  auto load_tile = [&](u32x4 *kd, u32x4 *vd, int t) {
    // one code path for both kinds of tile (a branch between two sets of
    // loads makes the compiler wait on the other set's registers); the base
    // and the clamp are scalar selects
    const bool full = whole(t);
    const int kbase = full ? t : min(t, kcap);
    const int klast = full ? t + TILE - 1 : kcap;
    const char *kb = ks + (size_t)kbase * ROWB;
    const char *vb = vs + (size_t)kbase * ROWB;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const uint32_t off = (uint32_t)(min(t + s * RPL + kr, klast) - kbase) * ROWB + ds * 16;
      kd[s] = load16(kb + off);
      vd[s] = load16(vb + off);
    }
    if constexpr (kRegNew) {
      if (t + TILE > nb0) {  // uniform: the tile holds new rows; every lane loads one (clamped)
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          const int r = min(max(t + s * RPL + kr - sp.new_base, 0), a.T_new - 1);
          const uint32_t off = (uint32_t)r * ROWB + ds * 16;
          nk[s] = load16(knb + off);
          nv[s] = load16(vnb + off);
        }
      }
    }
  };
  auto load_a = [&](int t) { load_tile(kA, vA, t); };
  // ---- the first tiles not loaded above go out now
  if (!early_a && t0 < kend) load_a(t0);
  if constexpr (PF == 2) {  // (each form measured fastest for its kernels)
    if (!early_b && t0 + stride < kend) load_tile(kB, vB, t0 + stride);
  }

  // ---- rotary cos / sin at the first row's position: no memory access, so
  // they are computed while the loads above are in flight
  float rc[ROPE ? VE : 1], rs[ROPE ? VE : 1];  // cos / sin at position rpos
  double thn[ROPE && FUSED ? VE : 1];           // exact angles of the lane's new-key pairs
  int rpos = -1;
  if constexpr (ROPE) {
    if constexpr (FUSED) {
      constexpr int HALF_VECS = kHeadDim / 2 / VE;  // the new-row loop's pair chunk is fixed per lane
#pragma unroll
      for (int e = 0; e < VE; ++e) thn[e] = rope_theta_at(a.rope_theta, (threadIdx.x % HALF_VECS) * VE + e);
    }
    rpos = sp.causal_base + row_id(a, bkv, hk, g0).i;
    rope_slice_cs<DT>(ds, rpos, RopeStep{a.rope_ratio}, rc, rs);
  }

  // ---- fused append: the new rows of this key range are rotated and
  // rounded once into LDS (the loop reads them there); row tile 0 also writes
  // them into the cache, after the key loop (a store counts in vmcnt with
  // the loads: issued here, every wait of the loop would wait for it too)
  __shared__ u32x4 s_new[(FUSED && !kRegNew) ? 2 * kMaxFusedRows * VPR : 1];
  if constexpr (FUSED && !kRegNew) {
    constexpr int HALF_VECS = kHeadDim / 2 / VE;
    const char *kn = static_cast<const char *>(a.k_new) + head * a.T_new * ROWB;
    const char *vn = static_cast<const char *>(a.v_new) + head * a.T_new * ROWB;
    const int n = (kspan - nb0) * HALF_VECS;
    for (int t = threadIdx.x; t < n; t += 64 * nw) {
      const int r = t / HALF_VECS, j = t % HALF_VECS;
      const int pos = nb0 + r;
      const size_t src = (size_t)(pos - sp.new_base) * ROWB;
      const PairChunks c = load_pair<DT, true>(kn + src, vn + src, j, pos, ROPE ? thn : nullptr);
      s_new[r * VPR + j] = c.klo;
      s_new[r * VPR + j + VPR / 2] = c.khi;
      s_new[(kMaxFusedRows + r) * VPR + j] = c.vlo;
      s_new[(kMaxFusedRows + r) * VPR + j + VPR / 2] = c.vhi;
    }
    __syncthreads();
  }

  // ---- query rows: rotate (fp32), fold in scale*log2(e)
  float qf[GM][VE];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
#pragma unroll
    for (int e = 0; e < VE; ++e) qf[g][e] = 0.f;
    if (g < gcount) {
      if constexpr (ROPE) {
        const RowId r = row_id(a, bkv, hk, g0 + g);
        const int pos = sp.causal_base + r.i;
        if (pos != rpos) {  // rows of one position share their cos / sin
          rope_slice_cs<DT>(ds, pos, RopeStep{a.rope_ratio}, rc, rs);
          rpos = pos;
        }
        rope_slice_f32<DT>(qraw[g], qpart[g], ds, rc, rs, qf[g]);
      } else {
        unpack16<DT>(qraw[g], qf[g]);
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) qf[g][e] *= a.scale_log2;
    }
  }

  float m[GM], l[GM], o[GM][VE];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) o[g][e] = 0.f;
  }

  // The new rows of the tile at t0 replace its loaded chunks, from LDS: a
  // uniform test per tile, then reads at clamped rows and a select per lane
  // (no branch around a read)
  auto overlay_new = [&](u32x4 *kv, u32x4 *vv) {
    if (t0 + TILE > nb0) {
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int key = t0 + s * RPL + kr;
        const int r = min(max(key - nb0, 0), kMaxFusedRows - 1);
        const u32x4 kn = s_new[r * VPR + ds], vn = s_new[(kMaxFusedRows + r) * VPR + ds];
        const bool fresh = key < kend && key >= nb0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kv[s][i] = fresh ? kn[i] : kv[s][i];
          vv[s][i] = fresh ? vn[i] : vv[s][i];
        }
      }
    }
  };

  // one tile: the keys [t0, t0 + TILE) of this wave, held in (kv, vv)
  auto step = [&](u32x4 *kv, u32x4 *vv) {
    if constexpr (FUSED && !kRegNew) overlay_new(kv, vv);
    float sc[kSteps][GM];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      float kf[VE];
      unpack16<DT>(kv[s], kf);
      const int key = t0 + s * RPL + kr;
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        sc[s][g] = -INFINITY;
        if (g < gcount) {  // uniform: every lane takes part in the DPP sum
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < VE; ++e) d = fmaf(qf[g][e], kf[e], d);
          d = group_sum<LPR>(d);
          if (key < lim[g] && key < kend) sc[s][g] = d;
        }
      }
    }
    float vf[kSteps][VE];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) unpack16<DT>(vv[s], vf[s]);
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      float mt = sc[0][g];
#pragma unroll
      for (int s = 1; s < kSteps; ++s) mt = fmaxf(mt, sc[s][g]);
      online_update(m[g], l[g], o[g], mt, [&](auto &&fn) {
#pragma unroll
        for (int s = 0; s < kSteps; ++s) fn(sc[s][g], vf[s]);
      });
    }
    // the buffer is free now (the conversions of the values fold into the
    // P.V instructions, so it is read until here): the tile PF strides ahead
    // goes out, PF - 1 tiles of math ahead of its use
    if (t0 + PF * stride < kend) load_tile(kv, vv, t0 + PF * stride);
    t0 += stride;
  };
  if constexpr (PF == 2) {
    while (t0 < kend) {
      step(kA, vA);
      if (t0 >= kend) break;
      step(kB, vB);
    }
  } else {
    // the same tile step written out on the one buffer (the compiler
    // schedules this form better than the step above called through pointers)
    while (t0 < kend) {
      if constexpr (FUSED) {
        // values past kend: p = 0 there must meet no Inf or NaN, and with
        // new rows the clamped row may be one not written yet (a select per
        // lane, no branch: a branch would cost register copies)
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          const bool in = t0 + s * RPL + kr < kend;
#pragma unroll
          for (int i = 0; i < 4; ++i) vA[s][i] = in ? vA[s][i] : 0u;
        }
      }
      if constexpr (BEAM) {  // the parent's cached rows into this beam's rows
        if (rt == 0) {
#pragma unroll
          for (int s = 0; s < kSteps; ++s) {
            const int key = t0 + s * RPL + kr;
            if (key < kend && key < nb0) {
              store16(kc + (size_t)key * ROWB + ds * 16, kA[s]);
              store16(vc + (size_t)key * ROWB + ds * 16, vA[s]);
            }
          }
        }
      }
      if constexpr (FUSED && !kRegNew) overlay_new(kA, vA);
      if constexpr (kRegNew) {
        // the tile's new rows over its clamped ones; row tile 0 writes them
        // into the cache (no load of this wave follows a tile with new rows
        // unless it has a single wave)
        if (t0 + TILE > nb0) {  // uniform
#pragma unroll
          for (int s = 0; s < kSteps; ++s) {
            const int key = t0 + s * RPL + kr;
            const bool fresh = key >= nb0 && key < kend;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              kA[s][i] = fresh ? nk[s][i] : kA[s][i];
              vA[s][i] = fresh ? nv[s][i] : vA[s][i];
            }
            if (rt == 0 && fresh) {
              store16(kc + (size_t)key * ROWB + ds * 16, nk[s]);
              store16(vc + (size_t)key * ROWB + ds * 16, nv[s]);
            }
          }
        }
      }
      float sc[kSteps][GM];
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        float kf[VE];
        unpack16<DT>(kA[s], kf);
        const int key = t0 + s * RPL + kr;
#pragma unroll
        for (int g = 0; g < GM; ++g) {
          sc[s][g] = -INFINITY;
          if (g < gcount) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < VE; ++e) d = fmaf(qf[g][e], kf[e], d);
            d = group_sum<LPR>(d);
            if (key < lim[g] && key < kend) sc[s][g] = d;
          }
        }
      }
      float vf[kSteps][VE];
#pragma unroll
      for (int s = 0; s < kSteps; ++s) unpack16<DT>(vA[s], vf[s]);
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        float mt = sc[0][g];
#pragma unroll
        for (int s = 1; s < kSteps; ++s) mt = fmaxf(mt, sc[s][g]);
        online_update(m[g], l[g], o[g], mt, [&](auto &&fn) {
#pragma unroll
          for (int s = 0; s < kSteps; ++s) fn(sc[s][g], vf[s]);
        });
      }
      // the buffer is free now (see the two-tile form above)
      t0 += stride;
      if (t0 < kend) load_a(t0);
    }
  }

  // ---- new rows past every query row of this tile (a row tile of early
  // queries sees only the first ones) are not in its tiles: row tile 0
  // copies them into the cache as they are
  if constexpr (kRegNew) {
    if (rt == 0) {
      const int from = max(kend, nb0);
      const int n = (kspan - from) * VPR;  // 16-byte chunks
      for (int t = threadIdx.x; t < n; t += 64 * nw) {
        const int key = from + t / VPR, j = t % VPR;
        const size_t src = (head * a.T_new + (size_t)(key - sp.new_base)) * ROWB + j * 16;
        const size_t dst = (size_t)key * ROWB + j * 16;
        store16(kc + dst, load16(static_cast<const char *>(a.k_new) + src));
        store16(vc + dst, load16(static_cast<const char *>(a.v_new) + src));
      }
    }
  }
  // ---- the fused append's cache writes (from LDS, which holds the rows as
  // rotated and rounded above)
  if constexpr (FUSED && !kRegNew) {
    if (rt == 0) {
      constexpr int HALF_VECS = kHeadDim / 2 / VE;
      const int n = (kspan - nb0) * HALF_VECS;
      for (int t = threadIdx.x; t < n; t += 64 * nw) {
        const int r = t / HALF_VECS, j = t % HALF_VECS;
        const int pos = nb0 + r;
        const PairChunks c{s_new[r * VPR + j], s_new[r * VPR + j + VPR / 2],
                           s_new[(kMaxFusedRows + r) * VPR + j], s_new[(kMaxFusedRows + r) * VPR + j + VPR / 2]};
        store_pair<DT>(kc + (size_t)pos * ROWB, vc + (size_t)pos * ROWB, j, c);
      }
    }
  }

  // ---- merge the key-row groups of the wave. With 8 lanes per key row and
  // 8 values per lane (16-bit caches), each exchange level splits the values
  // (a lane keeps one half and adds its partner's copy of that half): lanes
  // 8 apart 8 -> 4, 16 apart 4 -> 2, 32 apart 2 -> 1, 7 exchanges instead of
  // 24, the same additions in the same pairs; every lane ends with one dim
  // of the wave's output (the rest of o is not read again).
  constexpr bool kSplitMerge = LPR == 8 && VE == 8;
  const bool upper = (lane & 8) != 0, upper16 = (lane & 16) != 0, upper32 = (lane & 32) != 0;
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    if (g < gcount) {
      const float M = groups_max<LPR>(m[g]);
      const float f = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[g] - M);
      l[g] = groups_sum<LPR>(l[g] * f);
      if constexpr (kSplitMerge) {
        float v4[4], v2[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // lanes 8 apart: 8 values -> 4
          const float lo_v = o[g][j] * f, hi_v = o[g][j + 4] * f;
          v4[j] = (upper ? hi_v : lo_v) + lane_xor8(upper ? lo_v : hi_v);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)  // lanes 16 apart: 4 -> 2
          v2[j] = (upper16 ? v4[j + 2] : v4[j]) + partner16(upper16 ? v4[j] : v4[j + 2], upper16);
        // lanes 32 apart: 2 -> 1, dim ds * VE + 4 * (lane bit 3) + 2 * (bit 4) + (bit 5)
        o[g][0] = (upper32 ? v2[1] : v2[0]) + partner32(upper32 ? v2[0] : v2[1], upper32);
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) o[g][e] = groups_sum<LPR>(o[g][e] * f);
      }
      m[g] = M;
    }
  }

  // ---- merge the waves in LDS; then write the rows (one workgroup per
  // tile) or publish the workgroup's partial and merge the splits
  __shared__ __attribute__((aligned(16))) float smem[NWMAX * GM * (D + 2)];
  float *sm_o = smem;                   // [nw][GM][D]
  float *sm_m = smem + NWMAX * GM * D;  // [nw][GM]
  float *sm_l = sm_m + NWMAX * GM;      // [nw][GM]
  if (kSplitMerge || kr == 0) {
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (g < gcount) {
        if constexpr (kSplitMerge) {
          sm_o[(wave * GM + g) * D + ds * VE + (upper ? 4 : 0) + (upper16 ? 2 : 0) + (upper32 ? 1 : 0)] = o[g][0];
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) sm_o[(wave * GM + g) * D + ds * VE + e] = o[g][e];
        }
        if (ds == 0 && kr == 0) {
          sm_m[wave * GM + g] = m[g];
          sm_l[wave * GM + g] = l[g];
        }
      }
    }
  }
  __syncthreads();
  const size_t tile_id = (size_t)unit * a.row_tiles + rt;
  float *part = a.ws_part + (tile_id * a.splits + split) * GM * kPStride;
  // output element idx (row idx / D, dim idx % D) of the tile: the waves'
  // (m, l, o) merged, then written or published as this split's partial
  auto finish = [&](int idx) {
    const int g = idx / D, d = idx % D;
    float mw[NWMAX], lw[NWMAX];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWMAX; ++w) {
      mw[w] = (w < nw) ? sm_m[w * GM + g] : -INFINITY;
      lw[w] = (w < nw) ? sm_l[w * GM + g] : 0.f;
      M = fmaxf(M, mw[w]);
    }
    // every slot is read (slots of absent waves hold stale values); a wave
    // with no keys or no slot contributes zeros
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NWMAX; ++w) {
      const bool ok = w < nw && mw[w] != -INFINITY;
      const float ow = sm_o[(w * GM + g) * D + d];
      const float f = ok ? __builtin_amdgcn_exp2f(mw[w] - M) : 0.f;
      Ls = fmaf(ok ? lw[w] : 0.f, f, Ls);
      O = fmaf(ok ? ow : 0.f, f, O);
    }
    if (a.splits == 1) {
      store_f32(a.out + orow[g] + d, O * __builtin_amdgcn_rcpf(Ls));
    } else {
      publish(part + g * kPStride + d, O);
      if (d == 0) {
        publish(part + g * kPStride + D, M);
        publish(part + g * kPStride + D + 1, Ls);
      }
    }
  };
  if (gcount * D <= 64) {
    // one wavefront holds the tile's output (one query row): it alone
    // publishes, waits for its stores, counts the arrival and, if last,
    // merges; the other waves are done, and no second barrier is needed
    if (wave != 0) return;
    if (lane < gcount * D) finish(lane);
    if (a.splits == 1) return;
    wait_stores();
    uint32_t *counter = a.ws_count + tile_id * kCounterStride;
    uint32_t prev = 0;
    if (lane == 0) prev = arrive(counter);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (uint32_t)(a.splits - 1)) return;
    if (lane == 0) reset_counter(counter);  // every split has arrived
    merge_rows<GM>(a, tile_id, a.splits, g0, gcount, bkv, hk, 0, 1);
    return;
  }
  for (int idx = threadIdx.x; idx < gcount * D; idx += 64 * nw) finish(idx);
  if (a.splits == 1) return;
  merge_splits<GM>(a, tile_id, g0, gcount, bkv, hk, nw);
}

template <int DT, bool FUSED, bool ROPE, bool RAGGED, bool BEAM>
void launch_gm(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  switch (a.gm) {
    case 1: launch_lead(attn_kernel<DT, 1, FUSED, 4, ROPE, RAGGED, BEAM>, grid, block, s, a); break;
    case 2: launch_lead(attn_kernel<DT, 2, FUSED, 4, ROPE, RAGGED, BEAM>, grid, block, s, a); break;
    case 4: launch_lead(attn_kernel<DT, 4, FUSED, 4, ROPE, RAGGED, BEAM>, grid, block, s, a); break;
    default:
      // fp32 tiles with rotary work stop at 4 rows (the plan's bucket): the
      // 8-row fused variant would not fit its registers
      if constexpr (DT == F32 && ROPE)
        launch_lead(attn_kernel<DT, 4, FUSED, 4, ROPE, RAGGED, BEAM>, grid, block, s, a);
      else
        launch_lead(attn_kernel<DT, 8, FUSED, 4, ROPE, RAGGED, BEAM>, grid, block, s, a);
      break;
  }
}

// The 8-wave variant (one wide workgroup per unit): one query row and no
// rotary work, so that it fits 128 registers without spilling.
template <int DT, bool FUSED, bool RAGGED, bool BEAM>
void launch_wide(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  launch_lead(attn_kernel<DT, 1, FUSED, kMaxWaves, false, RAGGED, BEAM>, grid, block, s, a);
}

template <int DT, bool FUSED, bool RAGGED, bool BEAM = false>
void launch_rg(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.waves > 4) launch_wide<DT, FUSED, RAGGED, BEAM>(a, grid, block, s);
  else if (a.rope_base > 0.f) launch_gm<DT, FUSED, true, RAGGED, BEAM>(a, grid, block, s);
  else launch_gm<DT, FUSED, false, RAGGED, BEAM>(a, grid, block, s);
}

template <int DT, bool FUSED>
void launch_dt(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  if constexpr (FUSED) {
    if (a.parent) {  // beam step (equal lengths)
      launch_rg<DT, true, false, true>(a, grid, block, s);
      return;
    }
  }
  if (a.lens) launch_rg<DT, FUSED, true>(a, grid, block, s);
  else launch_rg<DT, FUSED, false>(a, grid, block, s);
}

// The testing hook's forced plan: one process-wide setting, read at every
// planning call; at rest (the default) nothing is forced.
std::atomic<int> g_force_mfma{-1}, g_force_waves{0}, g_force_chunk{0};

}  // namespace

PlanOverride plan_override() {
  return PlanOverride{g_force_mfma.load(std::memory_order_relaxed),
                      g_force_waves.load(std::memory_order_relaxed),
                      g_force_chunk.load(std::memory_order_relaxed)};
}

void set_plan_override(PlanOverride o) {
  g_force_mfma.store(o.mfma, std::memory_order_relaxed);
  g_force_waves.store(o.waves, std::memory_order_relaxed);
  g_force_chunk.store(o.chunk, std::memory_order_relaxed);
}

// Matrix-core tile plan (blocks of queries, 16-bit storage): 16-row tiles;
// four tiles per workgroup and one split when there are enough tiles to fill
// the chip (prefill), else one tile per workgroup with its 4 or 8 waves
// sharing its keys and the keys split like the streaming kernel's.
AttnPlan plan_attn_mfma(int units, int G, int L, bool rope) {
  constexpr int kRows = 16, kStep = 32;
  AttnPlan p{};
  p.mfma = 1;
  p.gm = kRows;
  p.waves = 4;
  const int tiles16 = (G + kRows - 1) / kRows;
  const long unit_bytes = (long)L * 2 * kHeadDim * 2;
  const PlanOverride ov = plan_override();
  const int forced = ov.chunk;
  // one 16-row tile per wave (prefill) needs 4 tiles per unit to keep the
  // workgroup's waves busy, and enough units to fill the chip; fewer rows
  // (verification) share one tile across the workgroup's waves
  if ((long)units * tiles16 >= 64 && tiles16 >= 4 && forced <= 0) {
    p.rw = 4;
    p.row_tiles = (tiles16 + 3) / 4;
    p.chunk = ((L + kStep - 1) / kStep) * kStep;
    p.splits = 1;
  } else {
    p.rw = 1;
    p.row_tiles = tiles16;
    const int min_chunk = kStep * 4;
    const size_t tiles = (size_t)units * p.row_tiles;
    // Without rotary work and with at most 256 tiles, a workgroup of 8 waves
    // keeps a unit of up to 128 KB of keys and values unsplit; otherwise the
    // limit is 64 KB on 4 waves, and the keys are split as in the streaming
    // plan. (GQA decode steps with rotary keys, 3 rows per tile and 24 units,
    // measured slower on 8 waves with every chunk tried, also after the
    // rotary values became shared: 6.95 us on 4 waves at length 768 against
    // 8.1-8.6 on 8.)
    const bool wide = !rope && tiles <= 256;
    int chunk = (unit_bytes <= (wide ? 128 : 64) * 1024) ? L : max(min_chunk, (L + 15) / 16);
    if (forced > 0) chunk = forced;
    chunk = ((chunk + min_chunk - 1) / min_chunk) * min_chunk;
    const int max_splits = kMaxSplits;
    int splits = (L + chunk - 1) / chunk;
    if (splits > max_splits) {
      chunk = (((L + max_splits - 1) / max_splits + min_chunk - 1) / min_chunk) * min_chunk;
      splits = (L + chunk - 1) / chunk;
    }
    // more tiles: wider chunks, so that 8-wave workgroups still number at
    // most 256 (cross attention of 4 sequences x 5 rows: 3 splits of 512
    // frames on 8 waves 10.6 us, against 11.3 for 6 splits of 256 on 4)
    if (wide && forced <= 0 && splits > 1 && tiles * splits > 256 && tiles <= 128) {
      const int target = (int)(256 / tiles);  // >= 2
      chunk = (((L + target - 1) / target + min_chunk - 1) / min_chunk) * min_chunk;
      splits = (L + chunk - 1) / chunk;
    }
    if (splits > 1 && tiles > (size_t)kMaxCounters) {
      chunk = ((L + min_chunk - 1) / min_chunk) * min_chunk;
      splits = 1;
    }
    p.chunk = chunk;
    p.splits = splits;
    // 8 waves there when every wave has a step and the workgroups number at
    // most 256. Measured, back-to-back periods, 5 rows per tile (5 drafts, or
    // 5 beams sharing the cross cache):
    // - self step, one sequence: unsplit on 8 waves at length 300 / 448 / 512
    //   6.08 / 6.67 / 6.78 us, against 7.09 / 7.2 / 7.55 split on 4 waves;
    //   up to 128 keys 4 waves stay ahead (4.28 against 4.46 us at 64);
    // - split chunks of 128 keys (every partial read in one round trip by the
    //   merge): self at 640 / 1024 on 4 waves 6.25 / 6.50 us, against 6.44 /
    //   6.67 on 8 waves of 128 and 6.73 / 6.83 on 8 waves of 256; cross
    //   attention over 1500 frames (12 splits) on 4 waves 6.72 us, against
    //   6.93 on 8 waves of 128 and 7.04 on 8 waves of 256 (6 splits);
    // - self step, 4 sequences (80 tiles) at length 448: unsplit on 8 waves
    //   7.4 us, against 8.4 split on 4 and 13.1 split on 8;
    // - cross attention over 1500 frames at B = 4 (480 workgroups): 11.4 us
    //   on 4 waves against 14.2 on 8;
    // - GQA decode steps with rotary keys at length 768: 6.95 -> 8.5 us.
    if (wide && chunk >= 8 * kStep && tiles * splits <= 256) p.waves = 8;
    if (ov.waves == 4 || (ov.waves == 8 && !rope)) p.waves = ov.waves;  // rotary: 4 waves
  }
  const size_t tiles = (size_t)units * p.row_tiles;
  p.part_floats = (p.splits > 1) ? tiles * p.splits * kRows * kPStride : 0;
  p.counters = tiles;
  return p;
}

hipError_t launch_attn(int dtype, const AttnArgs &a, hipStream_t s) {
  if (a.mfma) return launch_attn_mfma(dtype, a, s);
  const dim3 grid(a.splits, a.row_tiles, a.Bkv * a.Hkv);
  const dim3 block(64 * a.waves);
  const bool fused = a.k_new != nullptr;
  switch (dtype) {
    case F32: fused ? launch_dt<F32, true>(a, grid, block, s) : launch_dt<F32, false>(a, grid, block, s); break;
    case F16: fused ? launch_dt<F16, true>(a, grid, block, s) : launch_dt<F16, false>(a, grid, block, s); break;
    default: fused ? launch_dt<BF16, true>(a, grid, block, s) : launch_dt<BF16, false>(a, grid, block, s); break;
  }
  return hipGetLastError();
}

// Split plan: a pure function of the shape (unless a test forces a plan
// through kvd_set_plan_override), so results are reproducible run to run.
// The thresholds come from timing back-to-back launches in a graph on
// MI355X: up to 96 KB of keys a unit stays on one workgroup (8 waves above
// 40 KB with one query row), which avoids the cross-workgroup merge (three
// memory round trips: the partial's stores, the arrival count, then the
// partials); beyond that the keys are split into chunks of at least 32 KB
// and at most 16 splits.
AttnPlan plan_attn(int dtype, int units, int G, int N, int L, bool rope, bool allow_mfma) {
  AttnPlan p{};
  // Matrix-core tiles for several query rows per KV head: N > 1 queries, or
  // G >= 3 rows from grouped heads or beams sharing one cache (measured: 3
  // GQA rows 12% and 5 beam rows 31% faster per decode step than 4- and 8-row
  // streaming tiles; 2 rows stay on the streaming kernel).
  const PlanOverride ov = plan_override();
  const bool use_mfma = allow_mfma && dtype != F32 && (N > 1 || G >= 3) && ov.mfma != 0;
  if (use_mfma) return plan_attn_mfma(units, G, L, rope);
  p.gm = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : (dtype == F32 && rope) ? 4 : 8;
  p.row_tiles = (G + p.gm - 1) / p.gm;
  const int tile = (dtype == F32) ? AttnGeom<F32>::TILE : AttnGeom<F16>::TILE;
  const int key_bytes = 2 * kHeadDim * ((dtype == F32) ? 4 : 2);  // K + V row
  const long unit_bytes = (long)L * key_bytes;
  const size_t tiles = (size_t)units * p.row_tiles;
  const bool wide_ok = p.gm == 1 && !rope;

  int waves = 4, chunk;
  if (tiles >= 256 || unit_bytes <= 96 * 1024) {
    chunk = L;  // one workgroup per (unit, row tile)
    if (tiles < 256 && unit_bytes > 32 * 1024 && wide_ok) waves = 8;  // measured (self, 1 row)
  } else {
    // at least 32 KB of keys per workgroup (one round of loads for 4 waves),
    // at most 16 splits. More workgroups pull more bandwidth (a few CUs
    // cannot stream a unit alone: the read probe over the 7.68 MB of one
    // cross-attention layer takes 4.3 us on 120 workgroups, 3.5 on 240 and
    // 2.9 on 960), and the merge reads every partial in one round trip, so
    // 1500 frames x 20 heads run as 12 splits of 128 on 4 waves: 5.67 us
    // back to back, against 6.10 for 6 splits of 256 on 8 waves and 6.06
    // to 6.74 for 24 to 47 splits of 1 or 2 waves (more arrivals per
    // counter, more partials)
    chunk = max((32 * 1024) / key_bytes, (L + 15) / 16);
    // a chunk that gives each of 4 waves an even number of tiles goes to 8
    // waves instead, same chunk (measured: 6 splits of 1500 frames, 6.02
    // against 6.21 us; with one tile per wave, 4 waves stay ahead)
    const int c4 = ((chunk + 4 * tile - 1) / (4 * tile)) * (4 * tile);
    if (wide_ok && c4 % (8 * tile) == 0) waves = 8;
  }
  if (ov.waves == 1 || ov.waves == 2 || ov.waves == 4 ||
      ((ov.waves == 8 || ov.waves == kMaxWaves) && wide_ok))
    waves = ov.waves;
  if (ov.chunk > 0) chunk = ov.chunk;
  p.waves = waves;

  const int min_chunk = tile * waves;
  const int max_splits = kMaxSplits;
  chunk = ((chunk + min_chunk - 1) / min_chunk) * min_chunk;
  if (chunk < min_chunk) chunk = min_chunk;
  int splits = (L + chunk - 1) / chunk;
  if (splits > max_splits) {  // too many partials to stage: widen the chunks
    chunk = (((L + max_splits - 1) / max_splits + min_chunk - 1) / min_chunk) * min_chunk;
    splits = (L + chunk - 1) / chunk;
  }
  if (splits > 1 && tiles > (size_t)kMaxCounters) {  // one counter per tile
    chunk = ((L + min_chunk - 1) / min_chunk) * min_chunk;
    splits = 1;
  }
  p.chunk = chunk;
  p.splits = splits;
  p.part_floats = (p.splits > 1) ? tiles * p.splits * p.gm * kPStride : 0;
  p.counters = tiles;
  return p;
}

}  // namespace kvd
