// moe_decode_host.hip -- host side of libmoe_decode.so: plan validation,
// workspace layout, kernel-variant choice and the launch sequence behind the
// C ABI of include/moe_decode.h.
//
// The forward follows the predicate-gated shape of the metrale page
// "forward_bf16_grouped_decode.rs" (fn forward_bf16_grouped_decode and
// bf16_grouped_decode_arena_ok): everything the kernels need is checked on
// the host first and an unsupported call returns an error having launched
// nothing; grids are sized for the worst case (cap = min(m*k, E) active
// experts) and the device-side active count trims the work, so the host never
// waits on the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "moe_decode.h"
#include "moe_kernels.hpp"
#include "moe_launch.hpp"

struct moe_decode_plan {
  moe_decode_desc d;
  moe_decode_ws_layout L;
  int variant;  // kSplit
  const moe::Variant *kv[moe::MAX_ROWS + 1];   // per m
  moe::launch_fn gate_up[moe::MAX_ROWS + 1];   // per m (split arrangement)
  moe::launch_fn gate_up_shd[moe::MAX_ROWS + 1];  // per m, with the shared down items
  bool route_in_gu[moe::MAX_ROWS + 1];         // per m: where the routing is computed
};

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status ok() {
  g_err.clear();
  return MOE_OK;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool log_enabled() {
  const char *v = getenv("MOE_DECODE_LOG");
  return v && v[0] == '1';
}

// Kernel arrangement: the work items as three launches ordered by the
// stream.  (A single persistent launch that chained the steps through
// completion words and bounded waits did not finish on MI355X; it was removed,
// and a plan asking for it with MOE_DECODE_VARIANT=fused is refused.)
constexpr int kSplit = 1;
const char *const kSplitStages[] = {"route", "gate_up", "down_blend"};
int num_stages(int) { return 3; }
const char *stage_name(int, int i) { return kSplitStages[i]; }

// Workgroups of the gate/up launch: a few per CU; each loops over items.
constexpr int kGateUpMaxBlocks = 1024;
// Compute units of MI355X, and the router units of a 16-wave route workgroup.
constexpr int kCUs = 256;
constexpr int kRouterUnitsWide = moe::ROUTE_THREADS_WIDE / moe::WAVE / moe::RSPLIT;

bool fused_requested() {
  const char *v = getenv("MOE_DECODE_VARIANT");
  return v && strcmp(v, "fused") == 0;
}

// Where a forward of m rows computes the routing.  For one row every gate/up
// workgroup computes it (from the logits, in LDS), which starts the expert
// streaming soonest; for more rows the router workgroup that finishes last
// computes it once and publishes it (the only placement the variants of
// m > 1 carry).  MOE_DECODE_ROUTE=once forces the published placement at
// m = 1 too (both give identical results; the tests run both).
bool route_in_gate_up(int m) {
  const char *v = getenv("MOE_DECODE_ROUTE");
  if (v && strcmp(v, "once") == 0) return false;
  return m == 1;
}

// Input vectors handled per pass over a weight tile: routed rows (pairs of
// one expert) and shared rows (all m rows); more are handled in further
// passes.  Restricted to the pairs the inst_*.hip tables instantiate.
void pass_variant(const moe_decode_desc &d, int m, int *cr, int *cs) {
  if (m == 1) { *cr = 1; *cs = 1; return; }
  if (d.act_fmt == MOE_F32) { *cr = 2; *cs = 2; return; }   // the fp32 path keeps two variants
  if (m <= 4) { *cr = 2; *cs = 4; return; }
  // Mean pairs per active expert (rounded up) plus one of headroom.  With
  // few pairs per expert, passes of up to 4 vectors: their down runs on 12
  // waves per workgroup (-5 to -6 % for the layer at m = 8-16).
  const int need = (m * d.top_k + d.num_experts - 1) / d.num_experts + 1;
  *cs = need <= 2 ? 4 : 8;
  *cr = need <= 2 ? 2 : 4;
}

// Lanes per down row: the smallest of 16/32/64 that covers the row's chunks
// without leaving most lanes idle.
int down_lanes(int chunks) {
  if (chunks <= 16) return 16;
  if (chunks <= 32) return 32;
  if (chunks < 128 && chunks % 64 != 0 && chunks % 32 == 0) return 32;
  return 64;
}

int elems_per_chunk(int fmt) { return fmt == MOE_F32 ? 4 : fmt == MOE_BF16 ? 8 : fmt == MOE_FP8_B128 ? 16 : 32; }

const moe::FormatKernels &kernels_for(int act, int ef) {
  typedef const moe::FormatKernels &(*getter)();
  static const getter t[2][6] = {
      {moe::kernels_f32_f32, moe::kernels_f32_bf16, moe::kernels_f32_aff4, moe::kernels_f32_mxfp4,
       moe::kernels_f32_nvfp4, moe::kernels_f32_fp8},
      {moe::kernels_bf16_f32, moe::kernels_bf16_bf16, moe::kernels_bf16_aff4, moe::kernels_bf16_mxfp4,
       moe::kernels_bf16_nvfp4, moe::kernels_bf16_fp8}};
  return t[act][ef]();
}

// Whether the shared expert runs on the matrix cores: bf16 activations with
// H and Is multiples of 32 (gate/up in the route launch, down in the gate/up
// launch); on the vector units otherwise.
bool shared_on_matrix_cores(const moe_decode_desc &d) {
  return (d.flags & MOE_SHARED) && d.act_fmt == MOE_BF16 && d.hidden % 32 == 0 && d.shared_inter % 32 == 0;
}


// Parts of K each routed down row is split into: up to 4 for long rows (at
// least 2048 elements each), so that one active expert still fills a tile's
// waves; fixed per layer (from max_rows, not m), so that a row's sums do not
// depend on m.  The parts' partial y share the down's LDS y array.
int down_parts_of(const moe_decode_desc &d) {
  int parts = 1;
  while (parts < 4 && d.inter / (2048 * (parts * 2)) >= 1 &&
         (size_t)d.max_rows * d.top_k * moe::MAX_DOWN_TILE * (parts * 2) <= (size_t)moe::MAX_PAIRS * moe::MAX_DOWN_TILE &&
         (d.inter / elems_per_chunk(d.expert_fmt)) % (parts * 2) == 0)
    parts *= 2;
  return parts;
}

// Narrow down tiles (4 waves, occupancy 4 per SIMD) resident at once on the
// 256 compute units.
constexpr int kNarrowResident = 4 * 256;

// The variant for m rows: the pass sizes pass_variant picks, with the lane
// grouping down_lanes wants if instantiated, else the widest available; at
// m = 1 the narrow down when a tile's sub-units (k experts times the parts of
// K) fit its 4 waves and it is instantiated.
bool pick_variant(const moe_decode_desc &d, int m, const moe::Variant **v, moe::launch_fn *gate_up,
                  moe::launch_fn *gate_up_shd) {
  int cr, cs;
  pass_variant(d, m, &cr, &cs);
  const int want = down_lanes(d.inter / elems_per_chunk(d.expert_fmt));
  const bool shared_vu = (d.flags & MOE_SHARED) && !shared_on_matrix_cores(d);
  const bool narrow = m == 1 && d.top_k * down_parts_of(d) + (shared_vu ? 1 : 0) <= 4;
  const moe::FormatKernels &k = kernels_for(d.act_fmt, d.expert_fmt);
  const moe::Variant *best = nullptr;
  // A narrow variant's tiles are c.narrow rows high: the lowest tiles whose
  // grid still fits one round of resident workgroups (a second round of a
  // few tiles would add a whole tile's latency at the end).
  auto fits = [&](const moe::Variant &c) { return (d.hidden + c.narrow - 1) / c.narrow <= kNarrowResident; };
  auto better = [&](const moe::Variant &c, const moe::Variant *b) {
    if (!b) return true;
    if ((c.lpr == want) != (b->lpr == want)) return c.lpr == want;
    if (c.lpr != b->lpr) return c.lpr > b->lpr;
    if (!c.narrow) return false;
    if (fits(c) != fits(*b)) return fits(c);
    return fits(c) ? c.narrow < b->narrow : c.narrow > b->narrow;
  };
  for (int pass = 0; pass < 2 && !best; ++pass)
  for (int i = 0; i < k.nv; ++i) {
    const moe::Variant &c = k.v[i];
    // First pass: a narrow variant where wanted; second: the others (no
    // narrow one instantiated).
    if (c.cr != cr || c.cs != cs || (pass == 0 && (c.narrow > 0) != narrow) || (pass == 1 && c.narrow)) continue;
    if (better(c, best)) best = &c;
  }
  *gate_up = *gate_up_shd = nullptr;
  for (int i = 0; i < k.ng; ++i)
    if (k.g[i].cr == cr && k.g[i].cs == cs) {
      *gate_up = k.g[i].gate_up;
      *gate_up_shd = m > 16 ? k.g[i].gate_up_shd2 : k.g[i].gate_up_shd;
    }
  *v = best;
  return best && *gate_up;
}

// Router rows of the route launch: the experts, plus the shared-expert gate
// vector unless the pre-norm launch takes it (router pre-norm).
int router_rows(const moe_decode_desc &d) {
  return d.num_experts + ((d.flags & MOE_SHARED_GATED) && !(d.flags & MOE_ROUTER_PRE_NORM) ? 1 : 0);
}

moe_status check_desc(const moe_decode_desc &d) {
  if (d.hidden <= 0 || d.num_experts <= 0 || d.top_k <= 0 || d.inter <= 0 || d.max_rows <= 0)
    return fail(MOE_EINVAL, "hidden, num_experts, top_k, inter and max_rows must be positive");
  if (d.act_fmt != MOE_F32 && d.act_fmt != MOE_BF16)
    return fail(MOE_EINVAL, "act_fmt must be MOE_F32 or MOE_BF16 (got %d)", d.act_fmt);
  if (d.expert_fmt < MOE_F32 || d.expert_fmt > MOE_FP8_B128)
    return fail(MOE_EINVAL, "unknown expert_fmt %d", d.expert_fmt);
  if (d.routing < MOE_ROUTE_SOFTMAX || d.routing > MOE_ROUTE_SQRTSOFTPLUS)
    return fail(MOE_EINVAL, "unknown routing %d", d.routing);
  const uint32_t known = MOE_NORM_TOPK | MOE_WEIGHT_BEFORE_FFN | MOE_SHARED | MOE_SHARED_GATED | MOE_OUT_F32 |
                         MOE_GEGLU | MOE_PRE_EXPERT_NORM | MOE_ROUTER_PRE_NORM;
  if (d.flags & ~known) return fail(MOE_EINVAL, "unknown flag bits 0x%x", d.flags & ~known);
  if ((d.flags & MOE_SHARED_GATED) && !(d.flags & MOE_SHARED))
    return fail(MOE_EINVAL, "MOE_SHARED_GATED requires MOE_SHARED");
  if (!std::isfinite(d.routed_scaling_factor))
    return fail(MOE_EINVAL, "routed_scaling_factor must be finite");
  if ((d.flags & (MOE_PRE_EXPERT_NORM | MOE_ROUTER_PRE_NORM)) && !(std::isfinite(d.norm_eps) && d.norm_eps >= 0.0f))
    return fail(MOE_EINVAL, "norm_eps must be finite and >= 0");
  if (d.num_experts > moe::MAX_EXPERTS)
    return fail(MOE_EUNSUPPORTED, "num_experts %d > %d", d.num_experts, moe::MAX_EXPERTS);
  if (d.top_k > d.num_experts || d.top_k > moe::MAX_TOPK)
    return fail(MOE_EUNSUPPORTED, "top_k %d must be <= min(num_experts, %d)", d.top_k, moe::MAX_TOPK);
  if (d.max_rows > moe::MAX_ROWS_G)
    return fail(MOE_EUNSUPPORTED, "max_rows %d > %d", d.max_rows, moe::MAX_ROWS_G);
  if (d.hidden % 8 || d.inter % 8)
    return fail(MOE_EUNSUPPORTED, "hidden and inter must be multiples of 8");
  if (d.expert_fmt == MOE_AFF4_G64 && (d.hidden % 64 || d.inter % 64))
    return fail(MOE_EUNSUPPORTED, "aff4-g64 experts need hidden and inter multiples of 64");
  if (d.expert_fmt == MOE_MXFP4_B32 && (d.hidden % 32 || d.inter % 32))
    return fail(MOE_EUNSUPPORTED, "mxfp4 experts need hidden and inter multiples of 32");
  if (d.expert_fmt == MOE_NVFP4_B16 && (d.hidden % 32 || d.inter % 32))
    return fail(MOE_EUNSUPPORTED, "nvfp4 experts need hidden and inter multiples of 32");
  if (d.expert_fmt == MOE_FP8_B128 && (d.hidden % 128 || d.inter % 128))
    return fail(MOE_EUNSUPPORTED, "fp8 experts need hidden and inter multiples of 128");
  if (d.flags & MOE_SHARED) {
    if (d.shared_inter <= 0 || d.shared_inter % 8)
      return fail(MOE_EUNSUPPORTED, "shared_inter must be a positive multiple of 8");
  }
  if (d.max_rows > moe::MAX_ROWS) {
    // The grouped path: bf16 matrix-core products over 32-wide k steps.
    if (d.act_fmt != MOE_BF16 || !kernels_for(d.act_fmt, d.expert_fmt).gate_up_grouped)
      return fail(MOE_EUNSUPPORTED, "max_rows above %d needs bf16 activations and bf16, 4-bit or fp8 experts",
                  moe::MAX_ROWS);
    if (d.hidden % 32 || d.inter % 32 || ((d.flags & MOE_SHARED) && d.shared_inter % 32))
      return fail(MOE_EUNSUPPORTED, "max_rows above %d needs hidden, inter and shared_inter multiples of 32",
                  moe::MAX_ROWS);
  }
  // Weight matrices are read through buffer resources with 32-bit byte
  // ranges: each projection (one expert's, or the shared expert's) must be
  // under 2 GiB.
  const double ebytes = d.expert_fmt == MOE_F32 ? 4.0 : d.expert_fmt == MOE_BF16 ? 2.0
                       : d.expert_fmt == MOE_FP8_B128 ? 1.0 : 0.5;
  const double abytes = d.act_fmt == MOE_F32 ? 4.0 : 2.0;
  const double lim = 2147483647.0;
  if ((double)d.hidden * d.inter * ebytes >= lim)
    return fail(MOE_EUNSUPPORTED, "an expert projection of %d x %d exceeds 2 GiB", d.inter, d.hidden);
  if ((d.flags & MOE_SHARED) && (double)d.hidden * d.shared_inter * abytes >= lim)
    return fail(MOE_EUNSUPPORTED, "a shared projection of %d x %d exceeds 2 GiB", d.shared_inter, d.hidden);
  return MOE_OK;
}

// Parts of Is that the matrix-core shared down splits across workgroups
// (about 2048 per part keeps every wave's stream short; at most
// MAX_SD_PARTS); 1 otherwise.  (Fewer parts on the 5120-wide layer -- one
// item per gate/up workgroup instead of 1.25 -- made its gate/up launch
// slower at m = 1 and 8: longer items.)
int shared_down_parts(const moe_decode_desc &d) {
  const int Is = (d.flags & MOE_SHARED) ? d.shared_inter : 0;
  const int p = Is / 2048;
  return p < 1 ? 1 : p > moe::MAX_SD_PARTS ? moe::MAX_SD_PARTS : p;
}

void layout_for(const moe_decode_desc &d, moe_decode_ws_layout *L) {
  const size_t A = 256;
  const size_t R = (size_t)d.max_rows, E = (size_t)d.num_experts;
  const size_t te = R * (size_t)d.top_k;
  const size_t cap = te < E ? te : E;
  const size_t Is = (d.flags & MOE_SHARED) ? (size_t)d.shared_inter : 0;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + (bytes ? bytes : 4), A);
    return at;
  };
  L->sync = take(moe::SYNC_WORDS * sizeof(uint32_t));
  L->logits = take(R * (E + 1) * sizeof(double));
  L->scores = take(d.routing == MOE_ROUTE_SQRTSOFTPLUS ? R * E * sizeof(double) : 0);
  L->topk_idx = take(te * 4);
  L->topk_w = take(te * 4);
  L->row_gate = take(R * 4);
  L->sorted_pair = take(te * 4);
  L->expert_offsets = take((E + 1) * 4);
  L->pair_to_perm = take(te * 4);
  L->active_experts = take(cap * 4);
  L->active_count = take(4);
  L->slot_info = take(cap * sizeof(moe::SlotRec));
  L->act = take(te * (size_t)d.inter * 4);
  L->shared_act = take(R * Is * 4);
  L->shared_y = take(Is ? (size_t)shared_down_parts(d) * R * (size_t)d.hidden * 4 : 0);
  L->routed_y = take(d.max_rows > moe::MAX_ROWS ? te * (size_t)d.hidden * 4 : 0);
  L->normed_x = take((d.flags & MOE_PRE_EXPERT_NORM) ? R * (size_t)d.hidden * (d.act_fmt == MOE_F32 ? 4 : 2) : 0);
  L->router_x = take((d.flags & MOE_ROUTER_PRE_NORM) ? R * (size_t)d.hidden * (d.act_fmt == MOE_F32 ? 4 : 2) : 0);
  L->total = o;
}

moe_status check_weights(const moe_decode_desc &d, const moe_decode_weights *w) {
  if (!w) return fail(MOE_EINVAL, "weights is NULL");
  if (!w->router_w || !aligned(w->router_w, 16))
    return fail(MOE_EINVAL, "router_w must be a non-null 16-byte aligned device pointer");
  if (!w->gate_w || !w->up_w || !w->down_w)
    return fail(MOE_EINVAL, "gate_w, up_w and down_w tables are required");
  if (d.expert_fmt >= MOE_AFF4_G64) {
    if (!w->gate_s || !w->up_s || !w->down_s)
      return fail(MOE_EINVAL, "4-bit and fp8 experts need gate_s, up_s and down_s tables");
  }
  if (d.expert_fmt == MOE_NVFP4_B16 && (!w->gate_scale2 || !w->up_scale2 || !w->down_scale2))
    return fail(MOE_EINVAL, "nvfp4 experts need gate_scale2, up_scale2 and down_scale2");
  if (d.expert_fmt == MOE_AFF4_G64 && (!w->gate_b || !w->up_b || !w->down_b))
    return fail(MOE_EINVAL, "aff4 experts need gate_b, up_b and down_b tables");
  if (d.routing == MOE_ROUTE_SIGMOID_BIAS && !w->expert_bias)
    return fail(MOE_EINVAL, "sigmoid+bias routing needs expert_bias");
  if (d.flags & MOE_SHARED) {
    if (!w->sh_gate_w || !w->sh_up_w || !w->sh_down_w || !aligned(w->sh_gate_w, 16) ||
        !aligned(w->sh_up_w, 16) || !aligned(w->sh_down_w, 16))
      return fail(MOE_EINVAL, "MOE_SHARED needs 16-byte aligned sh_gate_w, sh_up_w, sh_down_w");
  }
  if ((d.flags & MOE_SHARED_GATED) && (!w->sh_gate_vec || !aligned(w->sh_gate_vec, 16)))
    return fail(MOE_EINVAL, "MOE_SHARED_GATED needs a 16-byte aligned sh_gate_vec");
  if ((d.flags & MOE_PRE_EXPERT_NORM) && (!w->pre_norm_w || !aligned(w->pre_norm_w, 16)))
    return fail(MOE_EINVAL, "MOE_PRE_EXPERT_NORM needs a 16-byte aligned pre_norm_w");
  if ((d.flags & MOE_ROUTER_PRE_NORM) && (!w->router_norm_w || !aligned(w->router_norm_w, 16)))
    return fail(MOE_EINVAL, "MOE_ROUTER_PRE_NORM needs a 16-byte aligned router_norm_w");
  return MOE_OK;
}

// m > 32: router units, top-k with the sort, then the grouped gate/up and
// down on the matrix cores and the blend (moe_kernels.hpp, grouped path).
// The three timed stages are route (router + top-k/sort), gate_up, and
// down_blend (down + blend).
moe_status forward_grouped(const moe_decode_plan_t *plan, moe::Args &a, void *stream, void *const *events,
                           hipEvent_t route_start) {
  const moe_decode_desc &d = plan->d;
  const moe::FormatKernels &k = kernels_for(d.act_fmt, d.expert_fmt);
  const int m = a.m;
  const bool shared = (d.flags & MOE_SHARED) != 0;
  a.route_in_gu = 1;
  // Router tiles: RT_E router rows x 8 input rows per unit.
  const int nrows = router_rows(d);
  a.n_router = (nrows + moe::RT_E - 1) / moe::RT_E * ((m + 7) / 8);
  a.n_router_wg = (a.n_router + moe::ROUTE_UNITS_PER_WG - 1) / moe::ROUTE_UNITS_PER_WG;
  a.n_shared_gu = 0;
  a.shared_mfma = 0;
  a.max_rows = d.max_rows;
  a.sd_parts = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto ev = [&](int i) -> hipEvent_t { return events ? static_cast<hipEvent_t>(events[i]) : nullptr; };
  hipError_t e;
  if ((e = moe::launch_route_tile(d.act_fmt, a, a.n_router_wg, s, route_start)) != hipSuccess)
    return fail(MOE_EHIP, "route launch: %s", hipGetErrorString(e));
  if ((e = moe::launch_topk_sort(a, (m + moe::ROUTE_WPB - 1) / moe::ROUTE_WPB, s, nullptr, ev(1))) != hipSuccess)
    return fail(MOE_EHIP, "top-k launch: %s", hipGetErrorString(e));
  const int gr = k.gu_grouped_rows;
  const int gu_items = moe::grouped_item_count(a.cap * ((d.inter + gr - 1) / gr), shared, (a.Is + gr - 1) / gr, m);
  if ((e = k.gate_up_grouped(a, gu_items, s, ev(2), ev(3))) != hipSuccess)
    return fail(MOE_EHIP, "gate_up launch: %s", hipGetErrorString(e));
  // Down rows of at most 2048: items of 64 columns on two waves (four for
  // aff4) that each take all four tiles over a part of K (an input fragment
  // serves four tiles); longer rows: items of 32 columns on eight waves, an
  // eighth of K each.
  const int kmax = d.inter > a.Is ? d.inter : a.Is;
  const bool wide = kmax <= 2048;
  const moe::launch_fn dn = wide ? k.down_grouped : k.down_grouped_long;
  const int cols = wide ? 16 * moe::G_DT : 16 * moe::G_DTL;
  const int dn_tiles = (d.hidden + cols - 1) / cols;
  const int dn_items = moe::grouped_item_count(a.cap * dn_tiles, shared, dn_tiles, m);
  if ((e = dn(a, dn_items, s, ev(4), nullptr)) != hipSuccess)
    return fail(MOE_EHIP, "down launch: %s", hipGetErrorString(e));
  const int bl_threads = m * (d.hidden / 4);
  if ((e = moe::launch_blend_grouped(a, (bl_threads + 255) / 256, s, nullptr, ev(5))) != hipSuccess)
    return fail(MOE_EHIP, "blend launch: %s", hipGetErrorString(e));
  return ok();
}

// The tag this call's slot records carry: a hash of its per-expert tables,
// expert input, workspace and row count, odd so that it is never the zero
// of a cleared record.  The kernels use a record only if it carries the tag.
int32_t call_tag(const moe::Args &a) {
  const uint64_t v[13] = {(uint64_t)(uintptr_t)a.gw, (uint64_t)(uintptr_t)a.uw, (uint64_t)(uintptr_t)a.dw,
                          (uint64_t)(uintptr_t)a.gs, (uint64_t)(uintptr_t)a.us, (uint64_t)(uintptr_t)a.ds,
                          (uint64_t)(uintptr_t)a.gb, (uint64_t)(uintptr_t)a.ub, (uint64_t)(uintptr_t)a.db,
                          (uint64_t)(uintptr_t)a.x, (uint64_t)(uintptr_t)a.sync, (uint64_t)a.m,
                          (uint64_t)(uint32_t)a.E};
  uint64_t h = 0x243F6A8885A308D3ull;
  for (int i = 0; i < 13; ++i) {
    h ^= v[i];
    h *= 0x9E3779B97F4A7C15ull;
    h ^= h >> 29;
  }
  return (int32_t)((uint32_t)(h >> 32) | 1u);
}

moe_status forward_impl(const moe_decode_plan_t *plan, const moe_decode_weights *w, const void *x,
                        int32_t m, void *out, int32_t *idx_out, float *w_out, void *workspace,
                        size_t workspace_bytes, void *stream, void *const *events, int32_t n_events) {
  if (!plan) return fail(MOE_EINVAL, "plan is NULL");
  const moe_decode_desc &d = plan->d;
  const moe_decode_ws_layout &L = plan->L;
  if (m < 1 || m > d.max_rows) return fail(MOE_EINVAL, "m = %d outside 1..max_rows (%d)", m, d.max_rows);
  if (!x || !aligned(x, 16)) return fail(MOE_EINVAL, "x must be a non-null 16-byte aligned device pointer");
  if (!out || !aligned(out, 16)) return fail(MOE_EINVAL, "out must be a non-null 16-byte aligned device pointer");
  if (!workspace) return fail(MOE_EWORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(MOE_EWORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(MOE_EWORKSPACE, "workspace has %zu bytes, the plan needs %zu", workspace_bytes, L.total);
  const int nst = num_stages(plan->variant);
  if (events && n_events != 2 * nst) return fail(MOE_EINVAL, "n_events must be %d", 2 * nst);
  moe_status st = check_weights(d, w);
  if (st != MOE_OK) return st;

  char *ws = static_cast<char *>(workspace);
  moe::Args a;
  memset(&a, 0, sizeof a);
  a.H = d.hidden;
  a.E = d.num_experts;
  a.K = d.top_k;
  a.I = d.inter;
  a.Is = (d.flags & MOE_SHARED) ? d.shared_inter : 0;
  a.m = m;
  a.te = m * d.top_k;
  a.cap = a.te < d.num_experts ? a.te : d.num_experts;
  a.act_fmt = d.act_fmt;
  a.expert_fmt = d.expert_fmt;
  a.routing = d.routing;
  a.flags = d.flags;
  a.rsf = d.routed_scaling_factor;
  a.x = x;
  a.xr = x;
  a.out = out;
  a.idx_out = idx_out;
  a.w_out = w_out;
  a.router = w->router_w;
  a.ebias = (d.routing == MOE_ROUTE_SIGMOID_BIAS || d.routing == MOE_ROUTE_SQRTSOFTPLUS) ? w->expert_bias : nullptr;
  a.gw = w->gate_w; a.uw = w->up_w; a.dw = w->down_w;
  a.gs = w->gate_s; a.us = w->up_s; a.ds = w->down_s;
  a.gb = w->gate_b; a.ub = w->up_b; a.db = w->down_b;
  if (d.expert_fmt == MOE_NVFP4_B16) {
    a.gs2 = w->gate_scale2; a.us2 = w->up_scale2; a.ds2 = w->down_scale2;
  }
  a.sgw = w->sh_gate_w; a.suw = w->sh_up_w; a.sdw = w->sh_down_w; a.sgv = w->sh_gate_vec;
  a.logits = reinterpret_cast<double *>(ws + L.logits);
  a.scores = reinterpret_cast<double *>(ws + L.scores);
  a.topk_idx = reinterpret_cast<int32_t *>(ws + L.topk_idx);
  a.topk_w = reinterpret_cast<float *>(ws + L.topk_w);
  a.row_gate = reinterpret_cast<float *>(ws + L.row_gate);
  a.sorted_pair = reinterpret_cast<int32_t *>(ws + L.sorted_pair);
  a.offsets = reinterpret_cast<int32_t *>(ws + L.expert_offsets);
  a.pair_to_perm = reinterpret_cast<int32_t *>(ws + L.pair_to_perm);
  a.active = reinterpret_cast<int32_t *>(ws + L.active_experts);
  a.active_count = reinterpret_cast<int32_t *>(ws + L.active_count);
  a.slots = reinterpret_cast<moe::SlotRec *>(ws + L.slot_info);
  a.act = reinterpret_cast<float *>(ws + L.act);
  a.sact = reinterpret_cast<float *>(ws + L.shared_act);
  a.sy = reinterpret_cast<float *>(ws + L.shared_y);
  a.y = reinterpret_cast<float *>(ws + L.routed_y);
  a.sync = reinterpret_cast<unsigned *>(ws + L.sync);
  // Pre-norms: the experts read the rows normed with the pre-expert norm, the
  // router the rows normed with the router pre-norm; one launch writes both
  // first (it opens the route stage's timing).
  hipEvent_t route_start = events ? static_cast<hipEvent_t>(events[0]) : nullptr;
  if (d.flags & (MOE_PRE_EXPERT_NORM | MOE_ROUTER_PRE_NORM)) {
    const bool pe = (d.flags & MOE_PRE_EXPERT_NORM) != 0, pr = (d.flags & MOE_ROUTER_PRE_NORM) != 0;
    void *xe = ws + L.normed_x, *xrn = ws + L.router_x;
    hipError_t e = moe::launch_pre_norm(d.act_fmt, a, x, pe ? w->pre_norm_w : nullptr,
                                        pr ? w->router_norm_w : nullptr, d.norm_eps, xe, xrn,
                                        static_cast<hipStream_t>(stream), route_start);
    if (e != hipSuccess) return fail(MOE_EHIP, "pre-norm launch: %s", hipGetErrorString(e));
    if (pe) a.x = xe;
    if (pr) a.xr = xrn;
    route_start = nullptr;
  }
  a.tag = call_tag(a);   // after a.x is final
  if (m > moe::MAX_ROWS) return forward_grouped(plan, a, stream, events, route_start);

  const moe::Variant &kv = *plan->kv[m];
  const int cr = kv.cr, cs = kv.cs, lpr = kv.lpr;
  const bool shared = (d.flags & MOE_SHARED) != 0;
  // Work items (each one 256-thread workgroup): see moe_kernels.hpp.
  const int wpb = moe::WPB;
  const int ni_s = 2;                                       // gate_up_ni<ACT>()
  const int nrb = (m + 7) / 8;                               // input-row blocks per router row
  a.route_in_gu = plan->route_in_gu[m] ? 1 : 0;
  a.n_router = router_rows(d) * nrb;   // router units
  // The shared expert runs on the matrix cores (16-row tiles, gate/up in the
  // route launch, down in the gate/up launch) for bf16 activations when H and
  // Is are multiples of 32; on the vector units otherwise.
  a.shared_mfma = shared_on_matrix_cores(d);
  // With bf16 experts the matrix-core shared activations travel as bf16
  // pairs (their shared down skips the per-item split); the other formats'
  // shared downs measured faster splitting f32.  A plan constant.
  a.sact_pairs = a.shared_mfma && d.expert_fmt == MOE_BF16 ? 1 : 0;
  const int ni_r = d.expert_fmt >= MOE_AFF4_G64 && cr == 1 ? 4 : 2;   // gate_up_ni<EF, CR>()
  a.max_rows = d.max_rows;
  a.sd_parts = shared_down_parts(d);
  if (a.shared_mfma) {
    a.n_shared_gu = (a.Is + 15) / 16;
    a.n_shared_dn = (d.hidden + 15) / 16 * a.sd_parts;
  } else {
    a.n_shared_gu = shared ? ((a.Is + ni_s - 1) / ni_s + moe::ROUTE_WPB - 1) / moe::ROUTE_WPB : 0;
    a.n_shared_dn = 0;
  }
  // Above 8 rows the route launch takes 16-wave workgroups (the routing's
  // top-k runs 16 rows at once) when they fit one round, one per CU: bf16
  // activations, and the shared expert, if any, on the matrix cores (two
  // of its 8-wave items per workgroup, the same sums).  Router units and
  // items compute the same values either way.
  const int router_wg_wide = (a.n_router + kRouterUnitsWide - 1) / kRouterUnitsWide;
  const int shared_wg_wide = a.shared_mfma ? (a.n_shared_gu + 1) / 2 : 0;
  const bool route_wide = m > 8 && d.act_fmt == MOE_BF16 && (a.shared_mfma || !shared) &&
                          router_wg_wide + shared_wg_wide <= kCUs;
  a.n_router_wg = route_wide ? router_wg_wide
                             : (a.n_router + moe::ROUTE_UNITS_PER_WG - 1) / moe::ROUTE_UNITS_PER_WG;
  const int route_blocks = a.n_router_wg + (route_wide ? shared_wg_wide : a.n_shared_gu);
  a.gu_items_per_slot = ((d.inter + ni_r - 1) / ni_r + wpb - 1) / wpb;
  a.n_routed_gu = a.cap * a.gu_items_per_slot;
  a.down_parts = down_parts_of(d);
  const int down_units = a.cap + (shared && !a.shared_mfma ? 1 : 0);
  // Two row blocks per tile when a tile's sub-units would leave waves idle
  // and the halved tile count still gives every CU a workgroup.
  const int down_waves = kv.down_threads / moe::WAVE;
  a.down_dq = (down_units * a.down_parts < down_waves && d.hidden / (2 * kv.rd) >= 256) ? 2 : 1;
  a.n_down = (d.hidden + kv.rd * a.down_dq - 1) / (kv.rd * a.down_dq);

  static thread_local bool logged = false;
  if (!logged && log_enabled()) {
    logged = true;
    fprintf(stderr,
            "[moe_decode] first forward: %s, m=%d H=%d E=%d k=%d I=%d Is=%d act=%d expert=%d "
            "routing=%d flags=0x%x | items: router %d, shared gate/up %d, routed gate/up %d "
            "(%d per slot), down %d (dq %d) | CR=%d CS=%d LPR=%d\n",
            "split", m, d.hidden, d.num_experts, d.top_k,
            d.inter, a.Is, d.act_fmt, d.expert_fmt, d.routing, d.flags, a.n_router, a.n_shared_gu,
            a.n_routed_gu, a.gu_items_per_slot, a.n_down, a.down_dq, cr, cs, lpr);
  }

  const moe::launch_fn gu = a.shared_mfma ? plan->gate_up_shd[m] : plan->gate_up[m];
  if (!gu) return fail(MOE_EUNSUPPORTED, "no gate_up variant for this shared-expert arrangement");
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto ev = [&](int i) -> hipEvent_t { return events ? static_cast<hipEvent_t>(events[i]) : nullptr; };
  hipError_t e;
  // The pass width only shapes the vector-unit shared gate/up; with the
  // matrix-core one the narrowest variant runs (fewest registers, so two
  // workgroups share a CU).
  const int route_cs = a.shared_mfma ? 1 : cs;
  if ((e = moe::launch_route(d.act_fmt, route_cs, a, route_blocks, s, route_start, ev(1), route_wide)) != hipSuccess)
    return fail(MOE_EHIP, "route launch: %s", hipGetErrorString(e));
  // gate_up: a grid-stride launch over the active slots' items.
  // With the routing computed in gate/up, one more workgroup publishes it.
  const int gu_items = a.n_routed_gu + a.n_shared_dn;
  const int gu_blocks = (gu_items < kGateUpMaxBlocks ? gu_items : kGateUpMaxBlocks) + a.route_in_gu;
  if ((e = gu(a, gu_blocks, s, ev(2), ev(3))) != hipSuccess)
    return fail(MOE_EHIP, "gate_up launch: %s", hipGetErrorString(e));
  if ((e = kv.down_blend(a, a.n_down, s, ev(4), ev(5))) != hipSuccess)
    return fail(MOE_EHIP, "down_blend launch: %s", hipGetErrorString(e));
  return ok();
}

// ------------------------------------------- the allocation-free forward
//
// Its workspace is a file-scope device array, one per GPU the library runs
// on, held until the process ends.  In host code `scratch` only names the
// array: its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept in g_scratch.  Every
// allocation-free call on a GPU shares that GPU's array, so such calls must
// not overlap there.  Its reserved words are cleared once, by a kernel, on
// the device's first call; every forward leaves them cleared.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // per device: the address of `scratch` there, or null

moe_status device_scratch(const moe_decode_plan_t *plan, hipStream_t stream, void **ws) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EUNSUPPORTED, "device %d past the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(MOE_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    e = moe::launch_clear_sync(reinterpret_cast<unsigned *>(static_cast<char *>(p) + plan->L.sync), moe::SYNC_WORDS,
                               stream);
    if (e != hipSuccess) return fail(MOE_EHIP, "scratch clear launch: %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ws = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_decode_plan(const moe_decode_desc *desc, moe_decode_plan_t **plan,
                           size_t *workspace_bytes) {
  if (!desc || !plan || !workspace_bytes) return fail(MOE_EINVAL, "desc, plan and workspace_bytes are required");
  *plan = nullptr;
  moe_status st = check_desc(*desc);
  if (st != MOE_OK) return st;
  moe_decode_plan_t *p = new (std::nothrow) moe_decode_plan_t;
  if (!p) return fail(MOE_EINVAL, "out of host memory");
  p->d = *desc;
  if (!(p->d.flags & MOE_SHARED)) p->d.shared_inter = 0;
  if (fused_requested()) {
    delete p;
    return fail(MOE_EUNSUPPORTED, "the single-launch arrangement is disabled");
  }
  p->variant = kSplit;
  for (int m = 1; m <= p->d.max_rows && m <= moe::MAX_ROWS; ++m) {
    if (!pick_variant(p->d, m, &p->kv[m], &p->gate_up[m], &p->gate_up_shd[m])) {
      delete p;
      return fail(MOE_EUNSUPPORTED, "no kernel variant for m = %d", m);
    }
    p->route_in_gu[m] = route_in_gate_up(m);
  }
  layout_for(p->d, &p->L);
  *plan = p;
  *workspace_bytes = p->L.total;
  return ok();
}

void moe_decode_plan_destroy(moe_decode_plan_t *plan) { delete plan; }

moe_status moe_decode_workspace_layout(const moe_decode_plan_t *plan, moe_decode_ws_layout *layout) {
  if (!plan || !layout) return fail(MOE_EINVAL, "plan and layout are required");
  *layout = plan->L;
  return ok();
}

moe_status moe_decode_workspace_init(const moe_decode_plan_t *plan, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  if (!plan) return fail(MOE_EINVAL, "plan is NULL");
  if (!workspace || !aligned(workspace, 256)) return fail(MOE_EWORKSPACE, "workspace must be non-null and 256-byte aligned");
  if (workspace_bytes < plan->L.total)
    return fail(MOE_EWORKSPACE, "workspace has %zu bytes, the plan needs %zu", workspace_bytes, plan->L.total);
  hipError_t e = moe::launch_clear_sync(reinterpret_cast<unsigned *>(static_cast<char *>(workspace) + plan->L.sync), moe::SYNC_WORDS,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EHIP, "workspace init launch: %s", hipGetErrorString(e));
  return ok();
}

moe_status moe_decode_forward(const moe_decode_plan_t *plan, const moe_decode_weights *w, const void *x,
                              int32_t m, void *out, int32_t *idx_out, float *w_out, void *workspace,
                              size_t workspace_bytes, void *stream) {
  return forward_impl(plan, w, x, m, out, idx_out, w_out, workspace, workspace_bytes, stream, nullptr, 0);
}

moe_status moe_decode_forward_noalloc(const moe_decode_plan_t *plan, const moe_decode_weights *w,
                                      const void *x, int32_t m, void *out, int32_t *idx_out, float *w_out,
                                      void *stream) {
  if (!plan) return fail(MOE_EINVAL, "plan is NULL");
  if (plan->L.total > kScratchBytes)
    return fail(MOE_EWORKSPACE,
                "the plan needs %zu bytes of workspace; the allocation-free forward holds %zu (use "
                "moe_decode_forward with a workspace of the caller's)",
                plan->L.total, kScratchBytes);
  void *ws = nullptr;
  moe_status st = device_scratch(plan, static_cast<hipStream_t>(stream), &ws);
  if (st != MOE_OK) return st;
  return forward_impl(plan, w, x, m, out, idx_out, w_out, ws, kScratchBytes, stream, nullptr, 0);
}

moe_status moe_decode_forward_timed(const moe_decode_plan_t *plan, const moe_decode_weights *w,
                                    const void *x, int32_t m, void *out, int32_t *idx_out, float *w_out,
                                    void *workspace, size_t workspace_bytes, void *stream,
                                    void *const *events, int32_t n_events) {
  if (!events) return fail(MOE_EINVAL, "events is NULL");
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return fail(MOE_EINVAL, "events[%d] is NULL", i);
  return forward_impl(plan, w, x, m, out, idx_out, w_out, workspace, workspace_bytes, stream, events,
                      n_events);
}

int32_t moe_decode_num_stages(const moe_decode_plan_t *plan) { return plan ? num_stages(plan->variant) : 0; }

const char *moe_decode_stage_name(const moe_decode_plan_t *plan, int32_t i) {
  if (!plan || i < 0 || i >= num_stages(plan->variant)) return "";
  return stage_name(plan->variant, i);
}

const char *moe_decode_last_error(void) { return g_err.c_str(); }

const char *moe_decode_version(void) { return "moe_decode 0.1 (gfx950)"; }

moe_status moe_decode_bench_copy(const void *src, void *dst, size_t bytes, void *stream) {
  if (!src || !dst || bytes % 16 || !aligned(src, 16) || !aligned(dst, 16))
    return fail(MOE_EINVAL, "bench_copy needs 16-byte aligned buffers and a multiple of 16 bytes");
  hipError_t e = moe::launch_bench_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EHIP, "bench_copy launch: %s", hipGetErrorString(e));
  return ok();
}

moe_status moe_decode_bench_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  if (!src || !sink || bytes % 16 || !aligned(src, 16))
    return fail(MOE_EINVAL, "bench_read needs a 16-byte aligned buffer, a multiple of 16 bytes and a sink");
  hipError_t e = moe::launch_bench_read(src, bytes, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EHIP, "bench_read launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
