// Host side of the C ABI declared in include/kamera.h: argument checks (no HIP call
// before they pass), kernel choice, launch on the caller's stream.
#include <stdint.h>
#include <string.h>

#include <cmath>
#include <cstdarg>
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "kamera.h"
#include "kamera_internal.h"

namespace {

thread_local std::string g_last_error;

kamera_status fail(kamera_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

kamera_status fail(kamera_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

enum Kernel { K_NONE = 0, K_ROTATE = 1, K_MFMA = 2, K_GENERIC = 3 };

constexpr int kMfmaMaxRank = 128;
constexpr int64_t kMaxTunedTokens = (int64_t)1 << 30;  // token ids stay in 32 bits

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Bytes of a KV element, and of a patch-factor element (bf16 for fp8 KV).
int64_t elem_bytes(int32_t dtype) { return dtype == KAMERA_BF16 ? 2 : dtype == KAMERA_FP8_E4M3 ? 1 : 4; }
int64_t factor_bytes(int32_t dtype) { return dtype == KAMERA_FP8_E4M3 ? 2 : elem_bytes(dtype); }

// Dtypes of the tuned kernels, and the alignment their vector accesses need (a lane
// moves 8 elements at once).
bool tuned_dtype(int32_t dtype) { return dtype == KAMERA_BF16 || dtype == KAMERA_FP8_E4M3; }
uintptr_t vec_align(int32_t dtype) { return dtype == KAMERA_FP8_E4M3 ? 8 : 16; }

// Exclusive end (bytes) of the KV memory a channel can touch, from its base.
// Returns false on int64 overflow.
bool kv_extent(const kamera_channel& c, int64_t layers, int64_t slots, int32_t page_size,
               int64_t pages, int64_t es, int64_t* out) {
  __int128 last = (__int128)(layers - 1) * c.layer_stride + (__int128)(c.heads - 1) * c.head_stride +
                  (c.dim - 1);
  if (page_size > 0)
    last += (__int128)(pages - 1) * c.page_stride + (__int128)(page_size - 1) * c.slot_stride;
  else
    last += (__int128)(slots - 1) * c.slot_stride;
  const __int128 end = (last + 1) * es;
  if (end > (__int128)INT64_MAX) return false;
  *out = (int64_t)end;
  return true;
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

struct Plan {
  int kernel[2] = {K_NONE, K_NONE};
  int launches = 0;
  int block_tokens = 0;
  int tiles_per_wave = 0;
  int rotate_unroll = 2;
  int valu = 0;  // rotate+patch in place: patch on VALU (measurement variant)
  int64_t units = 0;  // workgroups of the tuned launch(es)
  // Pool order: with a workspace of pool_bytes, the rotate+patch launch sweeps the paged
  // pool in page order through the inverse of the block table (0: not applicable).
  int64_t pool_bytes = 0;
  int pool_block_tokens = 0;  // tokens (pool slots) one pool-order workgroup covers
};

bool strides_ok(const kamera_channel& c) {
  return c.layer_stride % 8 == 0 && c.slot_stride % 8 == 0 && c.head_stride % 8 == 0 &&
         c.page_stride % 8 == 0;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest element offset inside one layer that a channel can touch, plus one.
__int128 layer_extent(const kamera_channel& c, int64_t T, int32_t page_size, int64_t pages) {
  __int128 last = (__int128)(c.heads - 1) * c.head_stride + (c.dim - 1);
  if (page_size > 0)
    last += (__int128)(pages - 1) * c.page_stride + (__int128)(page_size - 1) * c.slot_stride;
  else
    last += (__int128)(T - 1) * c.slot_stride;
  return last + 1;
}

// Rotation-only kernel: 8-element lanes over the rotated dims of each row.
bool rotate_tuned_ok(const kamera_kv_desc& kv, const kamera_channel& c, int64_t T) {
  const int r = c.rope_dim;
  // one layer is reached through a buffer resource with 32-bit byte offsets
  const bool extent_ok = layer_extent(c, T, kv.page_size, kv.num_pages) * elem_bytes(kv.dtype) <=
                         kamera::kMaxBufferBytes;
  return tuned_dtype(kv.dtype) && !(kv.flags & KAMERA_FLAG_GENERIC) &&
         (r == 16 || r == 32 || r == 64 || r == 128) && T < kMaxTunedTokens && extent_ok &&
         aligned(c.data, vec_align(kv.dtype)) && strides_ok(c);
}

// Rotate+patch kernel: 128-feature blocks hold whole heads (or whole blocks of one
// head), a NeoX partner sits r/16 lanes away, rank <= 128 (fp8: a multiple of 8).
bool mfma_tuned_ok(const kamera_kv_desc& kv, const kamera_channel& c, const kamera_patch& p,
                   int ci, int64_t T) {
  const int r = c.rope_dim, D = c.dim;
  const bool rope_ok = r == 0 || ((r == 16 || r == 32 || r == 64 || r == 128) && D % r == 0);
  const bool dim_ok = D % 8 == 0 && (D % 128 == 0 || 128 % D == 0);
  // one layer of the channel and one layer of U are each reached through a buffer
  // resource with 32-bit byte offsets
  const bool extent_ok =
      layer_extent(c, T, kv.page_size, kv.num_pages) * elem_bytes(kv.dtype) <=
          kamera::kMaxBufferBytes &&
      (__int128)T * p.rank * factor_bytes(kv.dtype) <= kamera::kMaxBufferBytes &&
      (__int128)c.heads * D * p.rank * factor_bytes(kv.dtype) <= kamera::kMaxBufferBytes;
  return tuned_dtype(kv.dtype) && !(kv.flags & KAMERA_FLAG_GENERIC) && p.rank <= kMfmaMaxRank &&
         (kv.dtype == KAMERA_BF16 || p.rank % 8 == 0) && rope_ok && dim_ok && extent_ok &&
         T < kMaxTunedTokens && aligned(c.data, vec_align(kv.dtype)) && aligned(p.U[ci], 16) &&
         aligned(p.V[ci], 16) && strides_ok(c) && (int64_t)c.heads * D < (1 << 24);
}


// Launch shape of the rotate+patch kernel for the channels in `use`.
void plan_mfma(const kamera_kv_desc& kv, const kamera_chunks& ch, int m, const bool* use,
               bool out_of_place, Plan* plan) {
  plan->launches++;
  // Each of the 4 wavefronts of a workgroup streams `tpw` 16-token tiles.  The
  // workgroup stages 8 KB of feature factor per 32 ranks once per chunk (and, paged, its
  // block-table entries), so larger ranks take more tiles per wave: 2 tiles at rank
  // <= 32, 4 at 64 with a paged cache, 2 at 64 with a contiguous one (the MLA-shaped
  // call: 0.212 ms with 4, 0.203 with 2; paged recall 4.11 ms with 4, 4.41 with 2; the
  // 72B paged call in logical order 4.22 with 4, 4.29 with 2).  fp8 rows carry half
  // the bytes, so fp8 takes twice the tiles (measured best).
  const int mk = std::max(1, (m + 31) / 32);
  const int per_mk = 2 * (mk == 3 ? 4 : mk);
  const bool fp8 = kv.dtype == KAMERA_FP8_E4M3;
  const int dflt = std::min(8, fp8 ? 2 * per_mk : (mk == 2 && kv.page_size == 0 ? 2 : per_mk));
  int tpw = env_int("KAMERA_TILES_PER_WAVE", dflt);
  if (tpw < 1 || tpw > kamera::kMaxBlockTokens / 64) tpw = dflt;
  plan->tiles_per_wave = tpw;
  plan->block_tokens = 64 * tpw;
  // The pool-order sweep needs no table lookup before its first loads, so its
  // workgroups start streaming sooner and shorter ones measured best: two tiles per wave
  // for bf16, three for fp8 (rows of half the bytes), each wave's whole share requested
  // together.
  const int pdflt = kv.dtype == KAMERA_FP8_E4M3 ? 3 : std::max(1, std::min(2, dflt));
  int ptpw = env_int("KAMERA_TILES_PER_WAVE", pdflt);
  if (ptpw < 1 || ptpw > kamera::kMaxBlockTokens / 64) ptpw = pdflt;
  plan->pool_block_tokens = 64 * ptpw;
  // KAMERA_PATCH_VALU=1 selects the VALU form of the patch (bf16 in place, rank <= 64)
  // for the MFMA-versus-VALU comparison; the tuned default is MFMA.
  plan->valu = env_int("KAMERA_PATCH_VALU", 0) != 0;
  // Token groups that chunk boundaries cut: in place, one more unit per boundary in the
  // same launch; out of place, or with more boundaries than groups, a second launch.
  const int64_t T = ch.total_tokens;
  const int64_t groups = ceil_div(T, plan->block_tokens);
  const int64_t tail_units =
      ch.num_chunks < 2 ? 0 : std::min<int64_t>((int64_t)ch.num_chunks - 1, groups);
  if (tail_units > 0 && (out_of_place || (int64_t)ch.num_chunks - 1 > groups)) plan->launches++;
  for (int c = 0; c < kv.num_channels; ++c)
    if (use[c])
      plan->units += (int64_t)kv.num_layers * (groups + tail_units) *
                     ceil_div((int64_t)kv.ch[c].heads * kv.ch[c].dim, 128);
}

// Checks every host-visible argument.  No HIP call is made here.
kamera_status validate(const kamera_kv_desc* kv, const kamera_chunks* ch, const kamera_patch* p,
                       Plan* plan) {
  if (!kv) return fail(KAMERA_E_NULL, "kv descriptor is NULL");
  if (!ch) return fail(KAMERA_E_NULL, "chunks descriptor is NULL");
  if (kv->dtype != KAMERA_BF16 && kv->dtype != KAMERA_F32 && kv->dtype != KAMERA_FP8_E4M3)
    return fail(KAMERA_E_UNSUPPORTED, "dtype %d is not bf16 (0), fp32 (1) or fp8 E4M3 (2)",
                kv->dtype);
  if (kv->pairing != KAMERA_NEOX_HALF && kv->pairing != KAMERA_INTERLEAVED)
    return fail(KAMERA_E_UNSUPPORTED, "pairing %d is not NeoX half-split (0) or interleaved (1)",
                kv->pairing);
  if (kv->num_sections < 0 || kv->num_sections > KAMERA_MAX_SECTIONS)
    return fail(KAMERA_E_SHAPE, "num_sections %d outside [0, %d]", kv->num_sections,
                KAMERA_MAX_SECTIONS);
  if (kv->reserved1 != 0) return fail(KAMERA_E_SHAPE, "kv.reserved1 must be 0");
  if (kv->flags & ~KAMERA_FLAG_GENERIC) return fail(KAMERA_E_SHAPE, "unknown flags 0x%x", kv->flags);
  if (kv->num_layers < 0) return fail(KAMERA_E_SHAPE, "num_layers %d < 0", kv->num_layers);
  if (kv->num_channels < 1 || kv->num_channels > 2)
    return fail(KAMERA_E_SHAPE, "num_channels %d is not 1 or 2", kv->num_channels);
  if (ch->num_chunks < 0) return fail(KAMERA_E_SHAPE, "num_chunks %d < 0", ch->num_chunks);
  if (ch->total_tokens < 0) return fail(KAMERA_E_SHAPE, "total_tokens < 0");
  if (ch->reserved0 != 0) return fail(KAMERA_E_SHAPE, "chunks.reserved0 must be 0");
  if (ch->num_chunks == 0 && ch->total_tokens != 0)
    return fail(KAMERA_E_SHAPE, "total_tokens > 0 with no chunks");
  if (ch->total_tokens >= ((int64_t)1 << 40)) return fail(KAMERA_E_SHAPE, "total_tokens too large");
  const int m = p ? p->rank : 0;
  if (p && p->reserved0 != 0) return fail(KAMERA_E_SHAPE, "patch.reserved0 must be 0");
  if (m < 0 || m > KAMERA_MAX_RANK)
    return fail(KAMERA_E_SHAPE, "rank %d outside [0, %d]", m, KAMERA_MAX_RANK);
  const int64_t es = elem_bytes(kv->dtype), fs = factor_bytes(kv->dtype);
  const bool empty = kv->num_layers == 0 || ch->total_tokens == 0;
  bool any_rope = false;
  for (int c = 0; c < kv->num_channels; ++c) {
    const kamera_channel& k = kv->ch[c];
    if (k.heads < 1 || k.dim < 1)
      return fail(KAMERA_E_SHAPE, "channel %d: heads %d and dim %d must be >= 1", c, k.heads, k.dim);
    if (k.rope_dim < 0 || k.rope_dim > k.dim || (k.rope_dim & 1))
      return fail(KAMERA_E_SHAPE, "channel %d: rope_dim %d must be even and in [0, dim=%d]", c,
                  k.rope_dim, k.dim);
    if (k.reserved0 != 0) return fail(KAMERA_E_SHAPE, "channel %d: reserved0 must be 0", c);
    if (k.layer_stride < 0 || k.slot_stride < 0 || k.head_stride < 0 || k.page_stride < 0)
      return fail(KAMERA_E_SHAPE, "channel %d: strides must be >= 0", c);
    if ((int64_t)k.heads * k.dim > ((int64_t)1 << 30))
      return fail(KAMERA_E_SHAPE, "channel %d: heads * dim too large", c);
    any_rope = any_rope || k.rope_dim > 0;
    if (!empty && !k.data) return fail(KAMERA_E_NULL, "channel %d: data is NULL", c);
    if (!aligned(k.data, es))
      return fail(KAMERA_E_ALIGN, "channel %d: data not aligned to %d bytes", c, (int)es);
    if (kv->dtype == KAMERA_FP8_E4M3) {
      if (!empty && !k.scale) return fail(KAMERA_E_NULL, "channel %d: fp8 with no scales", c);
      if (!aligned(k.scale, 4)) return fail(KAMERA_E_ALIGN, "channel %d: scales not 4-byte aligned", c);
    }
  }
  if (any_rope && !(std::isfinite(kv->rope_theta) && kv->rope_theta > 0))
    return fail(KAMERA_E_SHAPE, "rope_theta must be finite and > 0");
  if (kv->num_sections > 1) {
    int sum = 0;
    for (int s = 0; s < kv->num_sections; ++s) {
      if (kv->section_pairs[s] < 0)
        return fail(KAMERA_E_SHAPE, "section_pairs[%d] = %d < 0", s, kv->section_pairs[s]);
      sum += kv->section_pairs[s];
    }
    for (int c = 0; c < kv->num_channels; ++c)
      if (kv->ch[c].rope_dim > 0 && sum != kv->ch[c].rope_dim / 2)
        return fail(KAMERA_E_SHAPE, "sections hold %d pairs but channel %d rotates %d", sum, c,
                    kv->ch[c].rope_dim / 2);
  }
  if (kv->page_size < 0) return fail(KAMERA_E_SHAPE, "page_size %d < 0", kv->page_size);
  if (kv->page_size > 0) {
    if (kv->num_pages < 1) return fail(KAMERA_E_SHAPE, "paged layout with num_pages < 1");
    if (!empty && !kv->block_table) return fail(KAMERA_E_NULL, "paged layout with no block table");
    if (!aligned(kv->block_table, 4)) return fail(KAMERA_E_ALIGN, "block table not 4-byte aligned");
  }
  if (!empty) {
    if (!ch->token_offsets) return fail(KAMERA_E_NULL, "token_offsets is NULL");
    if (!ch->delta) return fail(KAMERA_E_NULL, "delta is NULL");
    if (!aligned(ch->token_offsets, 8) || !aligned(ch->delta, 8))
      return fail(KAMERA_E_ALIGN, "token_offsets / delta not 8-byte aligned");
  }
  if (m > 0) {
    for (int c = 0; c < kv->num_channels; ++c) {
      if (!empty && (!p->U[c] || !p->V[c]))
        return fail(KAMERA_E_NULL, "channel %d: rank %d with a NULL factor", c, m);
      if (!aligned(p->U[c], fs) || !aligned(p->V[c], fs))
        return fail(KAMERA_E_ALIGN, "channel %d: factor not aligned to %d bytes", c, (int)fs);
    }
  }
  // Factors must not overlap any KV memory the call writes.
  if (m > 0 && !empty) {
    for (int c = 0; c < kv->num_channels; ++c) {
      int64_t kend;
      if (!kv_extent(kv->ch[c], kv->num_layers, ch->total_tokens, kv->page_size, kv->num_pages, es,
                     &kend))
        return fail(KAMERA_E_SHAPE, "channel %d: KV extent overflows", c);
      for (int f = 0; f < kv->num_channels; ++f) {
        const int64_t F = (int64_t)kv->ch[f].heads * kv->ch[f].dim;
        const __int128 ub = (__int128)kv->num_layers * ch->total_tokens * m * fs;
        const __int128 vb = (__int128)kv->num_layers * ch->num_chunks * F * m * fs;
        if (ub > INT64_MAX || vb > INT64_MAX) return fail(KAMERA_E_SHAPE, "factor size overflows");
        if (overlaps(kv->ch[c].data, kend, p->U[f], (int64_t)ub) ||
            overlaps(kv->ch[c].data, kend, p->V[f], (int64_t)vb))
          return fail(KAMERA_E_ALIAS, "factors of channel %d overlap KV of channel %d", f, c);
      }
    }
  }

  // Kernel choice.
  if (empty) return KAMERA_OK;
  const int64_t T = ch->total_tokens;
  if (m == 0) {
    for (int c = 0; c < kv->num_channels; ++c) {
      const kamera_channel& k = kv->ch[c];
      if (k.rope_dim == 0) continue;
      plan->kernel[c] = rotate_tuned_ok(*kv, k, T) ? K_ROTATE : K_GENERIC;
      plan->launches++;
      if (plan->kernel[c] == K_ROTATE) {
        // A workgroup covers 4 waves x `unroll` row groups of 64 / (rope_dim / 8) rows.
        // Interleaved rows keep more values live per row group: two groups fit the
        // register budget of four waves per SIMD, four would spill.
        // fp8 rows hold half the registers: four or eight groups (eight measured best).
        const bool q8 = kv->dtype == KAMERA_FP8_E4M3;
        const int udflt = q8 ? 8 : kv->pairing == KAMERA_INTERLEAVED ? 2 : 4;
        int unroll = env_int("KAMERA_ROTATE_UNROLL", udflt);
        if (q8 ? (unroll != 4 && unroll != 8) : (unroll != 2 && unroll != 4)) unroll = udflt;
        const int rows = 4 * unroll * (64 / (k.rope_dim / 8));
        const int bt = (int)std::min<int64_t>(kamera::kMaxBlockTokens,
                                              std::max<int64_t>(1, rows / k.heads));
        plan->rotate_unroll = unroll;
        plan->block_tokens = bt;
        plan->units += (int64_t)kv->num_layers * ceil_div(T, bt);
      }
    }
    return KAMERA_OK;
  }
  bool use[2] = {false, false};
  for (int c = 0; c < kv->num_channels; ++c) {
    use[c] = mfma_tuned_ok(*kv, kv->ch[c], *p, c, T);
    plan->kernel[c] = use[c] ? K_MFMA : K_GENERIC;
    if (!use[c]) plan->launches++;
  }
  if (use[0] || use[1]) {
    plan_mfma(*kv, *ch, m, use, false, plan);
    // Pool order: one chunk over a paged cache whose pages are multiples of 16 slots
    // (each 16-token tile lies in one page) and whose pool is at most four times the
    // pages the chunk uses (the sweep visits every pool page).
    const int P = kv->page_size;
    const int64_t lpages = P > 0 ? ceil_div(T, P) : 0;
    if (P > 0 && P % 16 == 0 && ch->num_chunks == 1 && kv->num_pages <= 4 * lpages &&
        env_int("KAMERA_POOL_ORDER", 1) != 0 && plan->valu == 0)
      plan->pool_bytes = (kv->num_pages * 4 + 255) / 256 * 256;
  }
  return KAMERA_OK;
}

kamera::CommonArgs common_args(const kamera_kv_desc& kv, const kamera_chunks& ch, int m, int bt) {
  kamera::CommonArgs a;
  memset(&a, 0, sizeof a);
  a.offsets = ch.token_offsets;
  a.delta = ch.delta;
  a.block_table = kv.block_table;
  a.total_tokens = ch.total_tokens;
  a.num_pages = kv.num_pages;
  a.block_tokens = bt > 0 ? bt : 64;
  a.token_groups = ceil_div(ch.total_tokens, a.block_tokens);
  a.theta = kv.rope_theta;
  a.num_chunks = ch.num_chunks;
  a.page_size = kv.page_size;
  a.num_layers = kv.num_layers;
  a.rank = m;
  a.page_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if (kv.page_size == (1 << sh)) a.page_shift = sh;
  a.out_page_shift = -1;
  a.pairing = kv.pairing;
  a.dtype = kv.dtype;
  a.num_sections = kv.num_sections > 1 ? kv.num_sections : 1;
  int end = 0;
  for (int s = 0; s < 4; ++s) {
    end += s < kv.num_sections ? kv.section_pairs[s] : 0;
    a.sec_end[s] = kv.num_sections > 1 ? end : (1 << 30);
  }
  return a;
}

kamera::ChanArgs chan_args(const kamera_kv_desc& kv, int ci, const kamera_patch* p) {
  const kamera_channel& c = kv.ch[ci];
  kamera::ChanArgs a;
  memset(&a, 0, sizeof a);
  a.data = c.data;
  a.layer_stride = c.layer_stride;
  a.slot_stride = c.slot_stride;
  a.head_stride = c.head_stride;
  a.page_stride = c.page_stride;
  a.U = p ? p->U[ci] : nullptr;
  a.V = p ? p->V[ci] : nullptr;
  a.scale = kv.dtype == KAMERA_FP8_E4M3 ? c.scale : nullptr;
  a.heads = c.heads;
  a.dim = c.dim;
  a.rope_dim = c.rope_dim;
  // Pair frequencies theta^(-2i/r) in fp64, the same expression the reference form uses.
  const int half = c.rope_dim / 2;
  for (int i = 0; i < half && i < kamera::kMaxTunedHalf; ++i)
    a.omega[i] = pow(kv.rope_theta, -2.0 * (double)i / (double)c.rope_dim);
  return a;
}

kamera_status hip_fail(hipError_t e, const char* what) {
  return fail(KAMERA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Checks a relocate workspace against the plan: big enough and aligned when the plan
// uses one, and clear of every buffer the call reads or writes.
kamera_status check_workspace(const kamera_kv_desc* kv, const kamera_chunks* ch,
                              const kamera_patch* p, const Plan& plan, const void* ws,
                              int64_t ws_bytes) {
  if (!ws || plan.pool_bytes == 0) return KAMERA_OK;
  if (ws_bytes < plan.pool_bytes)
    return fail(KAMERA_E_SHAPE, "workspace of %lld bytes; this call needs %lld",
                (long long)ws_bytes, (long long)plan.pool_bytes);
  if (!aligned(ws, 16)) return fail(KAMERA_E_ALIGN, "workspace not 16-byte aligned");
  const int m = p ? p->rank : 0;
  const int64_t es = elem_bytes(kv->dtype), fs = factor_bytes(kv->dtype);
  const int64_t T = ch->total_tokens, n = ch->num_chunks;
  for (int c = 0; c < kv->num_channels; ++c) {
    int64_t kend = 0;
    if (kv_extent(kv->ch[c], kv->num_layers, T, kv->page_size, kv->num_pages, es, &kend) &&
        overlaps(kv->ch[c].data, kend, ws, plan.pool_bytes))
      return fail(KAMERA_E_ALIAS, "workspace overlaps KV of channel %d", c);
    if (m > 0) {
      const int64_t F = (int64_t)kv->ch[c].heads * kv->ch[c].dim;
      if (overlaps(p->U[c], (int64_t)kv->num_layers * T * m * fs, ws, plan.pool_bytes) ||
          overlaps(p->V[c], (int64_t)kv->num_layers * n * F * m * fs, ws, plan.pool_bytes))
        return fail(KAMERA_E_ALIAS, "workspace overlaps the factors of channel %d", c);
    }
  }
  const int S = kv->num_sections > 1 ? kv->num_sections : 1;
  if (overlaps(kv->block_table, ceil_div(T, kv->page_size) * 4, ws, plan.pool_bytes) ||
      overlaps(ch->token_offsets, (n + 1) * 8, ws, plan.pool_bytes) ||
      overlaps(ch->delta, n * S * 8, ws, plan.pool_bytes))
    return fail(KAMERA_E_ALIAS, "workspace overlaps the block table, offsets or deltas");
  return KAMERA_OK;
}

kamera_status run(const kamera_kv_desc* kv, const kamera_chunks* ch, const kamera_patch* p,
                  void* ws, int64_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  Plan plan;
  kamera_status st = validate(kv, ch, p, &plan);
  if (st != KAMERA_OK) return st;
  if (ws_bytes < 0) return fail(KAMERA_E_SHAPE, "workspace_bytes < 0");
  st = check_workspace(kv, ch, p, plan, ws, ws_bytes);
  if (st != KAMERA_OK || plan.launches == 0) return st;
  const int m = p ? p->rank : 0;
  const bool pool = ws != nullptr && plan.pool_bytes > 0;
  kamera::CommonArgs cm = common_args(*kv, *ch, m, pool ? plan.pool_block_tokens : plan.block_tokens);
  if (pool) {
    cm.inv = (const int32_t*)ws;
    cm.num_logical_pages = ceil_div(ch->total_tokens, kv->page_size);
    cm.pool_slots = kv->num_pages * kv->page_size;
    cm.token_groups = ceil_div(cm.pool_slots, cm.block_tokens);
    const hipError_t e = kamera::launch_table_inverse(kv->block_table, cm.num_logical_pages,
                                                      kv->num_pages, (int32_t*)ws, stream);
    if (e != hipSuccess) return hip_fail(e, "block-table inverse launch");
  }
  if (m == 0) {
    for (int c = 0; c < kv->num_channels; ++c) {
      if (plan.kernel[c] == K_NONE) continue;
      kamera::ChanArgs a = chan_args(*kv, c, nullptr);
      a.layer_bytes = (uint32_t)(layer_extent(kv->ch[c], ch->total_tokens, kv->page_size,
                                              kv->num_pages) *
                                 elem_bytes(kv->dtype));
      const hipError_t e = plan.kernel[c] == K_ROTATE
                               ? kamera::launch_rotate_rows(a, cm, plan.rotate_unroll, stream)
                                                      : kamera::launch_generic(a, cm, kv->dtype, stream);
      if (e != hipSuccess) return hip_fail(e, "rotation launch");
    }
    return KAMERA_OK;
  }
  kamera::ChanArgs tuned[2];
  int ntuned = 0;
  for (int c = 0; c < kv->num_channels; ++c) {
    kamera::ChanArgs a = chan_args(*kv, c, p);
    if (plan.kernel[c] == K_MFMA) {
      const int64_t T = ch->total_tokens;
      a.layer_bytes = (uint32_t)(layer_extent(kv->ch[c], T, kv->page_size, kv->num_pages) *
                                 elem_bytes(kv->dtype));
      a.u_layer_bytes = (uint32_t)(T * m * factor_bytes(kv->dtype));
      a.fblocks = (int)ceil_div((int64_t)a.heads * a.dim, 128);
      a.blocks = cm.token_groups * a.fblocks;
      tuned[ntuned++] = a;
    } else {
      const hipError_t e = kamera::launch_generic(a, cm, kv->dtype, stream);
      if (e != hipSuccess) return hip_fail(e, "generic launch");
    }
  }
  if (ntuned > 0) {
    const hipError_t e =
        kamera::launch_relocate_patch_rows(tuned, ntuned, cm, plan.valu, pool, stream);
    if (e != hipSuccess) return hip_fail(e, "relocate+patch launch");
  }
  return KAMERA_OK;
}

// Out-of-place (recall) kernel: the rotate+patch kernel with a destination layout;
// ranks that are multiples of 8 (0 included), both layouts 16-byte addressable.
bool recall_tuned_ok(const kamera_kv_desc& src, const kamera_kv_desc& dst, const kamera_patch* p,
                     int ci, int64_t T) {
  const kamera_channel& c = src.ch[ci];
  const kamera_channel& d = dst.ch[ci];
  const int m = p ? p->rank : 0;
  const int r = c.rope_dim, D = c.dim;
  const bool rope_ok = r == 0 || ((r == 16 || r == 32 || r == 64 || r == 128) && D % r == 0);
  const bool dim_ok = D % 8 == 0 && (D % 128 == 0 || 128 % D == 0);
  const int64_t es = elem_bytes(src.dtype);
  const bool extent_ok =
      layer_extent(c, T, src.page_size, src.num_pages) * es <= kamera::kMaxBufferBytes &&
      layer_extent(d, T, dst.page_size, dst.num_pages) * es <= kamera::kMaxBufferBytes &&
      (__int128)T * m * factor_bytes(src.dtype) <= kamera::kMaxBufferBytes &&
      (__int128)c.heads * D * m * factor_bytes(src.dtype) <= kamera::kMaxBufferBytes;
  const bool factors_ok = m == 0 || (aligned(p->U[ci], 16) && aligned(p->V[ci], 16));
  const uintptr_t va = vec_align(src.dtype);
  return tuned_dtype(src.dtype) && !((src.flags | dst.flags) & KAMERA_FLAG_GENERIC) &&
         m <= kMfmaMaxRank && m % 8 == 0 && rope_ok && dim_ok && extent_ok &&
         T < kMaxTunedTokens && aligned(c.data, va) && aligned(d.data, va) && factors_ok &&
         strides_ok(c) && strides_ok(d) && (int64_t)c.heads * D < (1 << 24);
}

// Checks every host-visible argument of a recall: the source side as for the in-place
// call, then the destination.  No HIP call is made here.
kamera_status validate_recall(const kamera_kv_desc* src, const kamera_kv_desc* dst,
                              const kamera_chunks* ch, const kamera_patch* p, Plan* plan) {
  Plan src_plan;
  const kamera_status st = validate(src, ch, p, &src_plan);
  if (st != KAMERA_OK) return st;
  if (!dst) return fail(KAMERA_E_NULL, "destination descriptor is NULL");
  if (dst->dtype != src->dtype)
    return fail(KAMERA_E_SHAPE, "destination dtype %d differs from source dtype %d", dst->dtype,
                src->dtype);
  if (dst->num_layers != src->num_layers || dst->num_channels != src->num_channels)
    return fail(KAMERA_E_SHAPE, "destination layers/channels differ from the source");
  if (dst->reserved1 != 0) return fail(KAMERA_E_SHAPE, "destination reserved1 must be 0");
  if (dst->flags & ~KAMERA_FLAG_GENERIC)
    return fail(KAMERA_E_SHAPE, "unknown destination flags 0x%x", dst->flags);
  const int64_t es = elem_bytes(src->dtype), fs = factor_bytes(src->dtype);
  const int m = p ? p->rank : 0;
  const int64_t T = ch->total_tokens;
  const bool empty = src->num_layers == 0 || T == 0;
  for (int c = 0; c < dst->num_channels; ++c) {
    const kamera_channel& d = dst->ch[c];
    const kamera_channel& k = src->ch[c];
    if (d.heads != k.heads || d.dim != k.dim || d.rope_dim != k.rope_dim)
      return fail(KAMERA_E_SHAPE, "destination channel %d: heads/dim/rope_dim differ", c);
    if (d.reserved0 != 0) return fail(KAMERA_E_SHAPE, "destination channel %d: reserved0 must be 0", c);
    if (d.layer_stride < 0 || d.slot_stride < 0 || d.head_stride < 0 || d.page_stride < 0)
      return fail(KAMERA_E_SHAPE, "destination channel %d: strides must be >= 0", c);
    if (!empty && !d.data) return fail(KAMERA_E_NULL, "destination channel %d: data is NULL", c);
    if (!aligned(d.data, es))
      return fail(KAMERA_E_ALIGN, "destination channel %d: data not aligned to %d bytes", c, (int)es);
  }
  if (dst->page_size < 0) return fail(KAMERA_E_SHAPE, "destination page_size %d < 0", dst->page_size);
  if (dst->page_size > 0) {
    if (dst->num_pages < 1) return fail(KAMERA_E_SHAPE, "paged destination with num_pages < 1");
    if (!empty && !dst->block_table)
      return fail(KAMERA_E_NULL, "paged destination with no block table");
    if (!aligned(dst->block_table, 4))
      return fail(KAMERA_E_ALIGN, "destination block table not 4-byte aligned");
  }
  if (empty) return KAMERA_OK;
  // The destination must not overlap the source or the factors.
  for (int c = 0; c < dst->num_channels; ++c) {
    int64_t dend;
    if (!kv_extent(dst->ch[c], dst->num_layers, T, dst->page_size, dst->num_pages, es, &dend))
      return fail(KAMERA_E_SHAPE, "destination channel %d: extent overflows", c);
    for (int f = 0; f < src->num_channels; ++f) {
      int64_t send;
      if (!kv_extent(src->ch[f], src->num_layers, T, src->page_size, src->num_pages, es, &send))
        return fail(KAMERA_E_SHAPE, "channel %d: KV extent overflows", f);
      if (overlaps(dst->ch[c].data, dend, src->ch[f].data, send))
        return fail(KAMERA_E_ALIAS, "destination channel %d overlaps source channel %d", c, f);
      if (m > 0) {
        const int64_t F = (int64_t)src->ch[f].heads * src->ch[f].dim;
        const int64_t ub = (int64_t)src->num_layers * T * m * fs;
        const int64_t vb = (int64_t)src->num_layers * ch->num_chunks * F * m * fs;
        if (overlaps(dst->ch[c].data, dend, p->U[f], ub) ||
            overlaps(dst->ch[c].data, dend, p->V[f], vb))
          return fail(KAMERA_E_ALIAS, "factors of channel %d overlap destination channel %d", f, c);
      }
    }
  }
  // Every channel is written whole, so every channel is launched.
  bool use[2] = {false, false};
  for (int c = 0; c < src->num_channels; ++c) {
    use[c] = recall_tuned_ok(*src, *dst, p, c, T);
    plan->kernel[c] = use[c] ? K_MFMA : K_GENERIC;
    if (!use[c]) plan->launches++;
  }
  if (use[0] || use[1]) plan_mfma(*src, *ch, m, use, true, plan);
  return KAMERA_OK;
}

int exact_log2(int v) {
  for (int sh = 0; sh < 31; ++sh)
    if (v == (1 << sh)) return sh;
  return -1;
}

kamera_status run_recall(const kamera_kv_desc* src, const kamera_kv_desc* dst,
                         const kamera_chunks* ch, const kamera_patch* p, hipStream_t stream) {
  g_last_error.clear();
  Plan plan;
  kamera_status st = validate_recall(src, dst, ch, p, &plan);
  if (st != KAMERA_OK || plan.launches == 0) return st;
  const int m = p ? p->rank : 0;
  kamera::CommonArgs cm = common_args(*src, *ch, m, plan.block_tokens);
  cm.out_block_table = dst->block_table;
  cm.out_num_pages = dst->num_pages;
  cm.out_page_size = dst->page_size;
  cm.out_page_shift = exact_log2(dst->page_size);
  kamera::ChanArgs tuned[2];
  int ntuned = 0;
  for (int c = 0; c < src->num_channels; ++c) {
    kamera::ChanArgs a = chan_args(*src, c, m > 0 ? p : nullptr);
    const kamera_channel& d = dst->ch[c];
    a.out = d.data;
    a.out_layer_stride = d.layer_stride;
    a.out_slot_stride = d.slot_stride;
    a.out_head_stride = d.head_stride;
    a.out_page_stride = d.page_stride;
    if (plan.kernel[c] == K_MFMA) {
      const int64_t T = ch->total_tokens, es = elem_bytes(src->dtype);
      a.layer_bytes =
          (uint32_t)(layer_extent(src->ch[c], T, src->page_size, src->num_pages) * es);
      a.out_layer_bytes = (uint32_t)(layer_extent(d, T, dst->page_size, dst->num_pages) * es);
      a.u_layer_bytes = (uint32_t)(T * m * factor_bytes(src->dtype));
      a.fblocks = (int)ceil_div((int64_t)a.heads * a.dim, 128);
      a.blocks = cm.token_groups * a.fblocks;
      tuned[ntuned++] = a;
    } else {
      const hipError_t e = kamera::launch_generic(a, cm, src->dtype, stream);
      if (e != hipSuccess) return hip_fail(e, "generic recall launch");
    }
  }
  if (ntuned > 0) {
    const hipError_t e =
        kamera::launch_relocate_patch_rows(tuned, ntuned, cm, plan.valu, false, stream);
    if (e != hipSuccess) return hip_fail(e, "recall launch");
  }
  return KAMERA_OK;
}

// ------------------------------------------------------------------ patch formation

constexpr int kFormBatch = 64;

int form_k(int m, int F) { return std::min(std::min((m + 17) & ~1, F), 128); }

int64_t form_problem_bytes(const kamera_form_desc& d, int c) {
  return 4 * kamera::form_workspace_floats(d.width[c], form_k(d.rank, d.width[c]));
}

kamera_status validate_form(const kamera_form_desc* d, const kamera_chunks* ch, bool* empty,
                            bool gram_only = false) {
  if (!d) return fail(KAMERA_E_NULL, "form descriptor is NULL");
  if (!ch) return fail(KAMERA_E_NULL, "chunks descriptor is NULL");
  if (d->dtype != KAMERA_BF16) return fail(KAMERA_E_UNSUPPORTED, "patch formation takes bf16 only");
  if (d->num_layers < 0) return fail(KAMERA_E_SHAPE, "num_layers %d < 0", d->num_layers);
  if (d->num_channels < 1 || d->num_channels > 2)
    return fail(KAMERA_E_SHAPE, "num_channels %d is not 1 or 2", d->num_channels);
  if (!gram_only && (d->rank < 1 || d->rank > KAMERA_FORM_MAX_RANK))
    return fail(KAMERA_E_SHAPE, "rank %d outside [1, %d]", d->rank, KAMERA_FORM_MAX_RANK);
  if (d->iterations < 0 || d->iterations > 64)
    return fail(KAMERA_E_SHAPE, "iterations %d outside [0, 64]", d->iterations);
  if (d->reserved0 != 0) return fail(KAMERA_E_SHAPE, "form.reserved0 must be 0");
  if (ch->num_chunks < 0 || ch->total_tokens < 0 || ch->reserved0 != 0)
    return fail(KAMERA_E_SHAPE, "bad chunks descriptor");
  if (ch->num_chunks == 0 && ch->total_tokens != 0)
    return fail(KAMERA_E_SHAPE, "total_tokens > 0 with no chunks");
  if (ch->total_tokens >= ((int64_t)1 << 31)) return fail(KAMERA_E_SHAPE, "total_tokens too large");
  *empty = d->num_layers == 0 || ch->total_tokens == 0;
  for (int c = 0; c < d->num_channels; ++c) {
    const int F = d->width[c];
    if (F < 64 || F > 1024 || F % 64 != 0)
      return fail(KAMERA_E_SHAPE, "channel %d: width %d is not a multiple of 64 in [64, 1024]", c, F);
    if (!*empty && (!d->delta[c] || (!gram_only && (!d->U[c] || !d->V[c]))))
      return fail(KAMERA_E_NULL, "channel %d: delta, U and V are required", c);
    if (!aligned(d->delta[c], 16))
      return fail(KAMERA_E_ALIGN, "channel %d: delta not 16-byte aligned", c);
    if (!aligned(d->U[c], 2) || !aligned(d->V[c], 2) || !aligned(d->sigma[c], 4))
      return fail(KAMERA_E_ALIGN, "channel %d: misaligned output", c);
  }
  if (!*empty && !ch->token_offsets) return fail(KAMERA_E_NULL, "token_offsets is NULL");
  if (!aligned(ch->token_offsets, 8)) return fail(KAMERA_E_ALIGN, "token_offsets not 8-byte aligned");
  return KAMERA_OK;
}

kamera_status run_form(const kamera_form_desc* d, const kamera_chunks* ch, void* ws, int64_t ws_bytes,
                       hipStream_t stream) {
  g_last_error.clear();
  bool empty = true;
  kamera_status st = validate_form(d, ch, &empty);
  if (st != KAMERA_OK || empty) return st;
  if (!ws) return fail(KAMERA_E_NULL, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(KAMERA_E_ALIGN, "workspace not 256-byte aligned");
  const int64_t T = ch->total_tokens, L = d->num_layers, n = ch->num_chunks, m = d->rank;
  // Outputs must not overlap the inputs, each other or the workspace.
  struct Range { const void* p; int64_t n; };
  Range in[5], out[6];
  int nin = 0, nout = 0;
  in[nin++] = {ws, ws_bytes};
  for (int c = 0; c < d->num_channels; ++c) {
    const int64_t F = d->width[c];
    in[nin++] = {d->delta[c], L * T * F * 2};
    out[nout++] = {d->U[c], L * T * m * 2};
    out[nout++] = {d->V[c], L * n * F * m * 2};
    if (d->sigma[c]) out[nout++] = {d->sigma[c], L * n * m * 4};
  }
  for (int a = 0; a < nout; ++a) {
    for (int b = 0; b < nin; ++b)
      if (overlaps(out[a].p, out[a].n, in[b].p, in[b].n))
        return fail(KAMERA_E_ALIAS, "a patch-formation output overlaps its input or the workspace");
    for (int b = a + 1; b < nout; ++b)
      if (overlaps(out[a].p, out[a].n, out[b].p, out[b].n))
        return fail(KAMERA_E_ALIAS, "patch-formation outputs overlap each other");
  }
  const int64_t problems = L * n;
  for (int c = 0; c < d->num_channels; ++c) {
    const int64_t per = form_problem_bytes(*d, c);
    if (ws_bytes < per)
      return fail(KAMERA_E_SHAPE, "workspace of %lld bytes holds no problem (needs %lld)",
                  (long long)ws_bytes, (long long)per);
  }
  for (int c = 0; c < d->num_channels; ++c) {
    kamera::FormArgs a;
    memset(&a, 0, sizeof a);
    a.delta = (const uint16_t*)d->delta[c];
    a.offsets = ch->token_offsets;
    a.ws = (float*)ws;
    a.U_out = (uint16_t*)d->U[c];
    a.V_out = (uint16_t*)d->V[c];
    a.sigma_out = d->sigma[c];
    a.total_tokens = T;
    a.num_chunks = (int32_t)n;
    a.F = d->width[c];
    a.k = form_k(d->rank, d->width[c]);
    a.m = d->rank;
    a.iters = d->iterations > 0 ? d->iterations : 8;
    a.num_layers = (int32_t)L;
    const int64_t batch = std::min<int64_t>({(int64_t)kFormBatch, problems,
                                             ws_bytes / form_problem_bytes(*d, c)});
    for (int64_t p0 = 0; p0 < problems; p0 += batch) {
      const int count = (int)std::min<int64_t>(batch, problems - p0);
      const hipError_t e = kamera::launch_form_batch(a, p0, count, stream);
      if (e != hipSuccess) return hip_fail(e, "patch-formation launch");
    }
  }
  return KAMERA_OK;
}

// ------------------------------------------------------------------ relocate-on-read attention

struct AttendPlan {
  int64_t splits = 0, split_tokens = 0, slots = 0, bytes = 0;
  int64_t qw_bytes = 0;  // prepared queries, first in the workspace (256-byte rounded)
  bool heads_mapping = false;  // one wave per KV head, a workgroup per (layer, split)
};

// Checks an attention call; no HIP call is made here.
kamera_status validate_attend(const kamera_kv_desc* kv, const kamera_chunks* ch,
                              const kamera_patch* p, const kamera_attend_desc* at,
                              AttendPlan* plan) {
  Plan ignored;
  const kamera_status st = validate(kv, ch, p, &ignored);
  if (st != KAMERA_OK) return st;
  if (!at) return fail(KAMERA_E_NULL, "attend descriptor is NULL");
  if (at->reserved0 != 0 || at->reserved1 != 0)
    return fail(KAMERA_E_SHAPE, "attend reserved fields must be 0");
  if (kv->num_channels != 2)
    return fail(KAMERA_E_UNSUPPORTED, "attention takes an MHA/GQA cache: channels K and V");
  const kamera_channel& K = kv->ch[0];
  const kamera_channel& V = kv->ch[1];
  if (kv->dtype != KAMERA_BF16 && kv->dtype != KAMERA_FP8_E4M3)
    return fail(KAMERA_E_UNSUPPORTED, "attention takes bf16 or fp8 E4M3 KV");
  const int es = kv->dtype == KAMERA_FP8_E4M3 ? 1 : 2;
  if (K.heads != V.heads || K.dim != V.dim)
    return fail(KAMERA_E_SHAPE, "K and V differ in heads or dim");
  if (K.dim != kamera::kAttendDim)
    return fail(KAMERA_E_UNSUPPORTED, "attention takes dim %d, not %d", kamera::kAttendDim, K.dim);
  if (V.rope_dim != 0) return fail(KAMERA_E_SHAPE, "the V channel does not rotate (rope_dim 0)");
  const int Hq = at->num_q_heads;
  if (Hq < 1 || Hq % K.heads != 0)
    return fail(KAMERA_E_SHAPE, "num_q_heads %d is not a multiple of the %d KV heads", Hq, K.heads);
  if (Hq / K.heads > kamera::kAttendMaxGroup)
    return fail(KAMERA_E_UNSUPPORTED, "more than %d query heads per KV head", kamera::kAttendMaxGroup);
  if (!std::isfinite(at->scale)) return fail(KAMERA_E_SHAPE, "scale must be finite");
  const int m = p ? p->rank : 0;
  if (m > 128 || m % 8 != 0)
    return fail(KAMERA_E_UNSUPPORTED, "attention takes ranks that are multiples of 8, up to 128");
  for (int c = 0; m > 0 && c < 2; ++c)
    if (!aligned(p->U[c], 16) || !aligned(p->V[c], 16))
      return fail(KAMERA_E_ALIGN, "channel %d: attention needs 16-byte aligned factors", c);
  const int64_t T = ch->total_tokens, L = kv->num_layers, n = ch->num_chunks;
  if (T >= kMaxTunedTokens) return fail(KAMERA_E_UNSUPPORTED, "total_tokens must be below 2^30");
  for (int c = 0; c < 2; ++c) {
    const kamera_channel& k = kv->ch[c];
    // rows start 16-byte aligned: strides of 8 bf16 or 16 fp8 elements
    const int64_t sa = 16 / es;
    if (!aligned(k.data, 16) || !strides_ok(k) || k.slot_stride % sa || k.head_stride % sa ||
        k.layer_stride % sa || k.page_stride % sa)
      return fail(KAMERA_E_ALIGN, "channel %d: attention needs 16-byte aligned rows", c);
    // rows are reached through buffer resources with 32-bit byte offsets
    if (layer_extent(k, T, kv->page_size, kv->num_pages) * es > kamera::kMaxBufferBytes)
      return fail(KAMERA_E_UNSUPPORTED, "channel %d: one layer spans 2^31 - 64 bytes or more", c);
  }
  if ((__int128)T * m * 2 > kamera::kMaxBufferBytes)
    return fail(KAMERA_E_UNSUPPORTED, "one layer of U spans 2^31 - 64 bytes or more");
  if (kv->page_size > 0 && ceil_div(T, kv->page_size) * 4 > kamera::kMaxBufferBytes)
    return fail(KAMERA_E_UNSUPPORTED, "block table of 2^29 entries or more");
  if (L > 0 && (!at->q || !at->out)) return fail(KAMERA_E_NULL, "q and out are required");
  if (!aligned(at->q, 4) || !aligned(at->out, 4) || !aligned(at->lse, 4))
    return fail(KAMERA_E_ALIGN, "q, out and lse must be 4-byte aligned");
  if (L == 0) return KAMERA_OK;
  // Splits: a 4-wave workgroup per (layer, KV head, split), 4096 of them, at least 1024
  // tokens each (a workgroup's setup and merge cost about as much as 16 tiles; measured:
  // fewer, longer splits on the Qwen-shaped call, 0.098 -> 0.076 ms, and no change on
  // the large calls).
  // With one wave per KV head a workgroup holds all heads of a split, and one such
  // workgroup fills a CU (8 waves of about 230 registers, two per SIMD), so
  // kAttendCus * (8 / heads) of them run at once.  The splits are as many as one round
  // of those holds: every workgroup then starts at once and walks a long range.
  // Measured with 8 KV heads: Llama-shaped call (32 layers) 2.15 ms at 64 splits, 2.12
  // at 24, 2.07 at 16, 2.05 at 8 (one round); 72B-shaped call (80 layers) 2.46 ms at 26
  // splits, 2.47 at 48, 2.20 at 16, 2.18 at 6, 2.17 at 3 (one round, 240 workgroups),
  // against 2.33 ms with 4-wave workgroups, so the mapping is the default with 8 KV
  // heads at ranks up to 64.  With 4 KV heads a workgroup is 4 waves and two fit a CU:
  // the Qwen-shaped call (28 layers, 4096 tokens) took 0.076 ms with 4-wave workgroups
  // per head (4 splits of 1024 tokens), 0.069 with this mapping at 18 splits and 0.064
  // at 9 (one workgroup per CU); with fp8 0.065, 0.061 at 18 and 0.072 at 9.  So bf16
  // counts one workgroup per CU and fp8 as many as fit; splits go down to 128 tokens.
  // KAMERA_ATTEND_HM=0/1 overrides (up to 8 heads).
  const bool hm_default = K.heads >= 4 && K.heads <= kamera::kAttendMaxHeadsPerGroup && m <= 64;
  plan->heads_mapping = K.heads <= kamera::kAttendMaxHeadsPerGroup &&
                        env_int("KAMERA_ATTEND_HM", hm_default ? 1 : 0) != 0;
  const int64_t units = L * K.heads;
  int64_t S;
  if (plan->heads_mapping) {
    const int64_t per_cu = kv->dtype == KAMERA_FP8_E4M3
                               ? std::max<int64_t>(1, kamera::kAttendMaxHeadsPerGroup / K.heads)
                               : 1;
    S = std::max<int64_t>(1, (int64_t)kamera::kAttendCus * per_cu / L);
    S = std::min<int64_t>(S, std::max<int64_t>(1, ceil_div(T, 128)));
  } else {
    S = std::max<int64_t>(1, ceil_div(4096, units));
    S = std::min<int64_t>(S, std::max<int64_t>(1, ceil_div(T, 1024)));
  }
  const int env_splits = env_int("KAMERA_ATTEND_SPLITS", 0);
  if (env_splits > 0) S = env_splits;
  if (T > 0) {
    int64_t TS = ceil_div(T, S);
    TS = ceil_div(TS, 32) * 32;
    S = ceil_div(T, TS);
    if (L * S * K.heads >= ((int64_t)1 << 31) || L * std::max<int64_t>(n, 1) * K.heads >= ((int64_t)1 << 31))
      return fail(KAMERA_E_UNSUPPORTED, "too many layers x heads x splits (or chunks) for one launch");
    plan->splits = S;
    plan->split_tokens = TS;
    plan->slots = S + std::max<int64_t>(n, 1) - 1;
    plan->qw_bytes = ceil_div(L * std::max<int64_t>(n, 1) * Hq * (kamera::kAttendDim + m) * 4, 256) * 256;
    plan->bytes = plan->qw_bytes + L * Hq * plan->slots * kamera::attend_slot_floats(m) * 4;
  }
  return KAMERA_OK;
}

kamera_status run_attend(const kamera_kv_desc* kv, const kamera_chunks* ch, const kamera_patch* p,
                         const kamera_attend_desc* at, void* ws, int64_t ws_bytes,
                         hipStream_t stream) {
  g_last_error.clear();
  AttendPlan plan;
  kamera_status st = validate_attend(kv, ch, p, at, &plan);
  if (st != KAMERA_OK || kv->num_layers == 0) return st;
  const int64_t L = kv->num_layers, T = ch->total_tokens, Hq = at->num_q_heads;
  const int m = p ? p->rank : 0;
  if (plan.bytes > 0) {
    if (!ws) return fail(KAMERA_E_NULL, "workspace is NULL");
    if (!aligned(ws, 16)) return fail(KAMERA_E_ALIGN, "workspace not 16-byte aligned");
    if (ws_bytes < plan.bytes)
      return fail(KAMERA_E_SHAPE, "workspace of %lld bytes is below the %lld needed",
                  (long long)ws_bytes, (long long)plan.bytes);
  }
  // Written buffers must not overlap each other or anything read.
  struct Range { const void* p; int64_t n; };
  Range w[3] = {{at->out, L * Hq * kamera::kAttendDim * 4},
                {at->lse, at->lse ? L * Hq * 4 : 0},
                {ws, plan.bytes}};
  Range r[7];
  int nr = 0;
  r[nr++] = {at->q, L * Hq * kamera::kAttendDim * 4};
  for (int c = 0; c < 2; ++c) {
    int64_t end = 0;
    if (!kv_extent(kv->ch[c], L, T, kv->page_size, kv->num_pages,
                   kv->dtype == KAMERA_FP8_E4M3 ? 1 : 2, &end))
      return fail(KAMERA_E_SHAPE, "channel %d: KV extent overflows", c);
    r[nr++] = {kv->ch[c].data, T > 0 ? end : 0};
    if (m > 0) {
      r[nr++] = {p->U[c], L * T * m * 2};
      r[nr++] = {p->V[c], L * ch->num_chunks * (int64_t)kv->ch[c].heads * kv->ch[c].dim * m * 2};
    }
  }
  for (int a = 0; a < 3; ++a) {
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(w[a].p, w[a].n, w[b].p, w[b].n))
        return fail(KAMERA_E_ALIAS, "out, lse and the workspace overlap");
    for (int b = 0; b < nr; ++b)
      if (overlaps(w[a].p, w[a].n, r[b].p, r[b].n))
        return fail(KAMERA_E_ALIAS, "out, lse or the workspace overlaps q, the cache or the factors");
  }
  kamera::AttendArgs a;
  memset(&a, 0, sizeof a);
  for (int c = 0; c < 2; ++c) {
    const kamera_channel& k = kv->ch[c];
    a.data[c] = k.data;
    a.layer_stride[c] = k.layer_stride;
    a.slot_stride[c] = k.slot_stride;
    a.head_stride[c] = k.head_stride;
    a.page_stride[c] = k.page_stride;
    a.U[c] = m > 0 ? p->U[c] : nullptr;
    a.V[c] = m > 0 ? p->V[c] : nullptr;
  }
  a.block_table = kv->block_table;
  a.num_pages = kv->num_pages;
  a.offsets = ch->token_offsets;
  a.delta = ch->delta;
  a.q = at->q;
  a.out = at->out;
  a.lse = at->lse;
  a.qw = (float*)ws;
  a.ws = ws ? (float*)((char*)ws + plan.qw_bytes) : nullptr;
  a.total_tokens = T;
  a.num_chunks = ch->num_chunks;
  a.num_sections = kv->num_sections > 1 ? kv->num_sections : 1;
  int end = 0;
  for (int s = 0; s < 4; ++s) {
    end += s < kv->num_sections ? kv->section_pairs[s] : 0;
    a.sec_end[s] = kv->num_sections > 1 ? end : (1 << 30);
  }
  a.pairing = kv->pairing;
  a.rope_dim = kv->ch[0].rope_dim;
  a.page_size = kv->page_size;
  a.num_layers = (int32_t)L;
  a.heads = kv->ch[0].heads;
  a.num_q_heads = (int32_t)Hq;
  a.group = (int32_t)(Hq / a.heads);
  a.rank = m;
  a.splits = (int32_t)plan.splits;
  a.split_tokens = (int32_t)plan.split_tokens;
  a.slots = (int32_t)plan.slots;
  a.slot_floats = kamera::attend_slot_floats(m);
  const int es = kv->dtype == KAMERA_FP8_E4M3 ? 1 : 2;
  a.fp8 = es == 1;
  for (int c = 0; c < 2; ++c) {
    a.layer_bytes[c] = (uint32_t)(layer_extent(kv->ch[c], T, kv->page_size, kv->num_pages) * es);
    a.kv_scale[c] = es == 1 ? kv->ch[c].scale : nullptr;
  }
  // The next tile's V rows go to a second LDS tile (more bytes in flight per wave, fewer
  // workgroups per CU): measured best at ranks 33-64, and no better or slower below;
  // KAMERA_ATTEND_DB=0/1 overrides.
  a.double_buffer = env_int("KAMERA_ATTEND_DB", m > 32 && m <= 64 ? 1 : 0) != 0;
  a.heads_mapping = plan.heads_mapping;
  a.scale_log2 = at->scale * 1.4426950408889634f;
  for (int i = 0; i < a.rope_dim / 2 && i < 64; ++i)
    a.omega[i] = pow(kv->rope_theta, -2.0 * (double)i / (double)a.rope_dim);
  const hipError_t e = kamera::launch_attend(a, stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return KAMERA_OK;
}

}  // namespace

extern "C" {

kamera_status kamera_attend_workspace(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                                      const kamera_patch* patch,
                                      const kamera_attend_desc* attend, int64_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(KAMERA_E_NULL, "bytes is NULL");
  *bytes = 0;
  AttendPlan plan;
  const kamera_status st = validate_attend(kv, chunks, patch, attend, &plan);
  if (st != KAMERA_OK) return st;
  *bytes = plan.bytes;
  return KAMERA_OK;
}

kamera_status kamera_attend(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                            const kamera_patch* patch, const kamera_attend_desc* attend,
                            void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return run_attend(kv, chunks, patch, attend, workspace, workspace_bytes, stream);
}

kamera_status kamera_form_workspace(const kamera_form_desc* desc, const kamera_chunks* chunks,
                                    int64_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(KAMERA_E_NULL, "bytes is NULL");
  *bytes = 0;
  bool empty = true;
  const kamera_status st = validate_form(desc, chunks, &empty);
  if (st != KAMERA_OK) return st;
  const int64_t problems = (int64_t)desc->num_layers * chunks->num_chunks;
  int64_t per = 0;
  for (int c = 0; c < desc->num_channels; ++c) per = std::max(per, form_problem_bytes(*desc, c));
  *bytes = empty ? 0 : per * std::min<int64_t>(kFormBatch, std::max<int64_t>(1, problems));
  return KAMERA_OK;
}

kamera_status kamera_form_patch(const kamera_form_desc* desc, const kamera_chunks* chunks,
                                void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return run_form(desc, chunks, workspace, workspace_bytes, stream);
}

kamera_status kamera_form_gram(const kamera_form_desc* desc, const kamera_chunks* chunks,
                               float* const G[2], hipStream_t stream) {
  g_last_error.clear();
  bool empty = true;
  kamera_status st = validate_form(desc, chunks, &empty, true);
  if (st != KAMERA_OK || empty) return st;
  if (!G) return fail(KAMERA_E_NULL, "G is NULL");
  const int64_t L = desc->num_layers, T = chunks->total_tokens, n = chunks->num_chunks;
  for (int c = 0; c < desc->num_channels; ++c) {
    const int64_t F = desc->width[c];
    if (!G[c]) return fail(KAMERA_E_NULL, "G[%d] is NULL", c);
    if (!aligned(G[c], 4)) return fail(KAMERA_E_ALIGN, "G[%d] not 4-byte aligned", c);
    for (int f = 0; f < desc->num_channels; ++f)
      if (overlaps(G[c], L * n * F * F * 4, desc->delta[f], L * T * desc->width[f] * 2))
        return fail(KAMERA_E_ALIAS, "G[%d] overlaps a deficit", c);
  }
  for (int c = 0; c < desc->num_channels; ++c) {
    kamera::FormArgs a;
    memset(&a, 0, sizeof a);
    a.delta = (const uint16_t*)desc->delta[c];
    a.offsets = chunks->token_offsets;
    a.total_tokens = T;
    a.num_chunks = (int32_t)n;
    a.num_layers = (int32_t)L;
    a.F = desc->width[c];
    const hipError_t e = kamera::launch_form_gram(a, G[c], stream);
    if (e != hipSuccess) return hip_fail(e, "Gram launch");
  }
  return KAMERA_OK;
}


kamera_status kamera_orbit_mean(const void* deltas, int32_t num_orders, int64_t elements,
                                int64_t order_stride, void* out, hipStream_t stream) {
  g_last_error.clear();
  if (num_orders < 1 || num_orders > (1 << 20))
    return fail(KAMERA_E_SHAPE, "num_orders %d outside [1, 2^20]", num_orders);
  if (elements < 0) return fail(KAMERA_E_SHAPE, "elements %lld < 0", (long long)elements);
  if (order_stride < elements)
    return fail(KAMERA_E_SHAPE, "order_stride %lld < elements %lld", (long long)order_stride,
                (long long)elements);
  if (order_stride > (INT64_MAX / 2) / num_orders)
    return fail(KAMERA_E_SHAPE, "num_orders * order_stride overflows");
  if (elements == 0) return KAMERA_OK;
  if (!deltas) return fail(KAMERA_E_NULL, "deltas is NULL");
  if (!out) return fail(KAMERA_E_NULL, "out is NULL");
  if (!aligned(deltas, 16) || !aligned(out, 16) || order_stride % 8 != 0)
    return fail(KAMERA_E_ALIGN, "deltas and out must be 16-byte aligned and order_stride a "
                                "multiple of 8");
  for (int64_t p = 0; p < num_orders; ++p)
    if (overlaps(out, elements * 2, (const uint16_t*)deltas + p * order_stride, elements * 2))
      return fail(KAMERA_E_ALIAS, "out overlaps the deficit of order %lld", (long long)p);
  const hipError_t e = kamera::launch_orbit_mean((const uint16_t*)deltas, num_orders, elements,
                                                 order_stride, (uint16_t*)out, stream);
  if (e != hipSuccess) return hip_fail(e, "orbit mean launch");
  return KAMERA_OK;
}

kamera_status kamera_recall_patch(const kamera_kv_desc* src, const kamera_kv_desc* dst,
                                  const kamera_chunks* chunks, const kamera_patch* patch,
                                  hipStream_t stream) {
  return run_recall(src, dst, chunks, patch, stream);
}

kamera_status kamera_recall_plan(const kamera_kv_desc* src, const kamera_kv_desc* dst,
                                 const kamera_chunks* chunks, const kamera_patch* patch,
                                 kamera_plan_info* out) {
  g_last_error.clear();
  if (!out) return fail(KAMERA_E_NULL, "plan output is NULL");
  memset(out, 0, sizeof *out);
  Plan plan;
  const kamera_status st = validate_recall(src, dst, chunks, patch, &plan);
  if (st != KAMERA_OK) return st;
  out->kernel[0] = plan.kernel[0];
  out->kernel[1] = plan.kernel[1];
  out->launches = plan.launches;
  out->tokens_per_unit = plan.block_tokens;
  out->units = plan.units;
  return KAMERA_OK;
}


kamera_status kamera_relocate(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                              hipStream_t stream) {
  return run(kv, chunks, nullptr, nullptr, 0, stream);
}

kamera_status kamera_relocate_patch(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                                    const kamera_patch* patch, hipStream_t stream) {
  return run(kv, chunks, patch, nullptr, 0, stream);
}

kamera_status kamera_relocate_patch_noalloc(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                                            const kamera_patch* patch, hipStream_t stream) {
  g_last_error.clear();
  Plan plan;
  const kamera_status st = validate(kv, chunks, patch, &plan);
  if (st != KAMERA_OK) return st;
  if (plan.pool_bytes > kamera::kScratchPoolPages * 4)
    return fail(KAMERA_E_SHAPE,
                "pool of %lld pages exceeds the library scratch of %lld pages "
                "(kamera_relocate_patch_ws takes any size)",
                (long long)kv->num_pages, (long long)kamera::kScratchPoolPages);
  if (plan.launches == 0 || plan.pool_bytes == 0) return run(kv, chunks, patch, nullptr, 0, stream);
  int32_t* ws = nullptr;
  const hipError_t e = kamera::scratch_inverse_table(stream, &ws);
  if (e != hipSuccess) return hip_fail(e, "scratch address lookup");
  return run(kv, chunks, patch, ws, plan.pool_bytes, stream);
}

kamera_status kamera_relocate_workspace(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                                        const kamera_patch* patch, int64_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(KAMERA_E_NULL, "bytes is NULL");
  *bytes = 0;
  Plan plan;
  const kamera_status st = validate(kv, chunks, patch, &plan);
  if (st != KAMERA_OK) return st;
  *bytes = plan.pool_bytes;
  return KAMERA_OK;
}

kamera_status kamera_relocate_patch_ws(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                                       const kamera_patch* patch, void* workspace,
                                       int64_t workspace_bytes, hipStream_t stream) {
  return run(kv, chunks, patch, workspace, workspace_bytes, stream);
}

kamera_status kamera_plan(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                          const kamera_patch* patch, kamera_plan_info* out) {
  g_last_error.clear();
  if (!out) return fail(KAMERA_E_NULL, "plan output is NULL");
  memset(out, 0, sizeof *out);
  Plan plan;
  const kamera_status st = validate(kv, chunks, patch, &plan);
  if (st != KAMERA_OK) return st;
  out->kernel[0] = plan.kernel[0];
  out->kernel[1] = plan.kernel[1];
  out->launches = plan.launches;
  out->tokens_per_unit = plan.block_tokens;
  out->units = plan.units;
  return KAMERA_OK;
}

const char* kamera_status_str(kamera_status s) {
  switch (s) {
    case KAMERA_OK: return "ok";
    case KAMERA_E_NULL: return "null pointer";
    case KAMERA_E_SHAPE: return "bad shape, stride, rank or rope_dim";
    case KAMERA_E_UNSUPPORTED: return "unsupported dtype or pairing";
    case KAMERA_E_ALIGN: return "misaligned pointer";
    case KAMERA_E_ALIAS: return "overlapping memory (factors and KV, or recall source and destination)";
    case KAMERA_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* kamera_last_error(void) { return g_last_error.c_str(); }

int kamera_abi_version(void) { return KAMERA_ABI_VERSION; }

}  // extern "C"
