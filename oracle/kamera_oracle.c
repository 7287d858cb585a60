/*
 * Kamera reuse operator: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load this library. The GPU library never links, includes
 * or calls it, and it shares no source with the GPU library.
 *
 * Sources cited below (web summaries of two papers):
 *   [K]  "Kamera: KV Cache Multimodal Unificado e Invariante a Posicao para Reuso
 *        sem Treinamento", gist.science/pt/paper/2606.23581, and its Korean twin
 *        at gist.science/ko/paper/2606.23581, which agrees on every point used here.
 *   [N]  "Modelos Tomam Notas no Prefill: O Cache KV Pode Ser Editavel e
 *        Componivel", gist.science/pt/paper/2606.17107.
 *
 * What the oracle computes, per layer l, channel c, chunk j, token t of chunk j,
 * head h and dim d of that head (feature f = h*D + d):
 *
 *     out = round( [R(delta_j) x](h, d)  +  sum_{k<m} U[l][t][k] * V[l][j][f][k] )
 *
 *   - [K §2, reuse equation]: the reused KV is the relocated canonical KV plus a
 *     rank-m patch U_m V_m^T, with U_m indexed by token and V_m by feature.
 *   - [K §2, "Relocacao"]: keys are turned by the RoPE phase shift of the new
 *     position; it is an exact rotation, not a network pass.
 *   - [K §2, architecture list]: MHA/GQA rotate the whole key; MLA rotates only
 *     the 64-dim decoupled k_rope and keeps c_KV as it is; the patch goes on
 *     both channels.
 *   - [K §3, sliding-window survival] and [N §3B, composable KV]: with no patch,
 *     only the keys move and the values are carried over unchanged.
 *
 * Readings taken where the pages are silent (the pages give no RoPE formula):
 *   - NeoX half-split pairing: rotary pair i (i < r/2) is dims (i, i + r/2), where
 *     r is the number of rotated dims of a head; dims >= r are not rotated.  The
 *     interleaved variant pairs dims (2i, 2i + 1) instead.
 *   - Pair frequency omega_i = theta^(-2i/r); angle delta * omega_i; the pair
 *     (a, b) turns to (a cos - b sin, b cos + a sin).  Positive delta moves the
 *     chunk to a later position.
 *   - Multimodal rotary positions (M-RoPE, named in [N §4, composition: image KV
 *     transplanted with M-RoPE re-rotation]): a position is a vector of up to 4
 *     components and the pairs are cut, in pair order, into as many sections; pair
 *     i of section s turns by delta[s] * omega_i.  A pair whose section delta is 0
 *     does not move.  One section is plain RoPE.
 *   - The patch is added after the rotation and is not itself rotated.
 *   - R(0) is the identity matrix: a chunk with delta 0 is not rotated at all.
 *   - The result is rounded once, from fp64, to the storage type (bf16 or fp32)
 *     with round-to-nearest-even.
 *   - 8-bit KV (the pages report the method holding on FP8-quantised models, [N
 *     closing summary]): elements are OCP FP8 E4M3 codes and channel c of layer l
 *     carries one dequantisation scale s, value = s * code value.  The operator
 *     acts on values: out = encode((R(delta) (s x) + U V^T) / s), where encode
 *     rounds to the nearest code, ties to the even one, and saturates at +-448.
 *     The factors stay bf16 (they are in value units).
 *   - With no patch (m = 0), elements the rotation does not move (channels with
 *     r = 0, dims >= r, chunks with delta = 0) keep their exact bits.
 *
 * Everything is plain loops over the definition; rows are independent, so an
 * OpenMP loop spreads rows over host threads without changing any arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BF16 0
#define ORC_F32 1
#define ORC_FP8 2 /* OCP FP8 E4M3 codes with a per-layer scale; factors in bf16 */

/* ---------------------------------------------------------------- numbers */

/* bf16 bits -> exact double value. */
double orc_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> bf16 bits, round to nearest, ties to even, straight from the double
 * (no detour through fp32, which would round twice).  bf16 keeps 8 significant
 * bits and the fp32 exponent range: normal numbers from 2^-126, subnormal
 * quantum 2^-133, largest finite (2 - 2^-7) * 2^127.  Reading [K §3,
 * production deployment]: the rebuilt KV is compared at bf16 rounding. */
uint16_t orc_bf16_from_double(double y) {
    uint16_t sign = signbit(y) ? 0x8000u : 0u;
    if (isnan(y)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(y)) return (uint16_t)(sign | 0x7F80u);
    double a = fabs(y);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                 /* a = f * 2^e, 0.5 <= f < 1 */
    int qexp = e - 8;             /* weight of the last kept bit */
    if (qexp < -133) qexp = -133; /* subnormal range: fixed quantum */
    double q = nearbyint(ldexp(a, -qexp)); /* default mode: ties to even */
    double r = ldexp(q, qexp);
    if (r >= 0x1p128) return (uint16_t)(sign | 0x7F80u);
    float rf = (float)r;          /* exact: r has <= 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &rf, sizeof bits);
    return (uint16_t)(sign | (bits >> 16));
}

void orc_round_bf16_array(const double* y, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_double(y[i]);
}

/* OCP 8-bit floating point, E4M3 variant (the fp8 KV type): bit 7 sign, bits 6..3
 * exponent with bias 7, bits 2..0 mantissa.  Exponent 0 holds the subnormals
 * mantissa * 2^-9; exponent field 15 with mantissa 7 is NaN; there are no
 * infinities, so exponent 15 with mantissa 0..6 is finite and 448 = 1.75 * 2^8 is
 * the largest value.  Code -> exact double. */
double orc_fp8_to_double(uint8_t b) {
    int e = (b >> 3) & 15, mt = b & 7;
    if (e == 15 && mt == 7) return NAN;
    double v = e == 0 ? ldexp((double)mt, -9) : ldexp((double)(8 + mt), e - 10);
    return (b & 0x80) ? -v : v;
}

/* Double -> E4M3 code: the nearest of the 127 finite magnitudes, a tie going to the
 * even code (mantissa bit 0 clear); magnitudes of 448 and above give 448
 * (saturation, no overflow to NaN); NaN gives NaN; the sign is kept, zero included.
 * Found by brute force over the magnitudes. */
uint8_t orc_fp8_from_double(double y) {
    uint8_t sign = signbit(y) ? 0x80 : 0;
    if (isnan(y)) return (uint8_t)(sign | 0x7F);
    double a = fabs(y);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int best = 0;
    double bd = a;
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(orc_fp8_to_double((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0)) { best = c; bd = d; }
    }
    return (uint8_t)(sign | best);
}

void orc_fp8_from_double_array(const double* y, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_from_double(y[i]);
}

/* Bytes of one element of the storage type, and the type of the patch factors. */
static int elem_size(int dtype) { return dtype == ORC_BF16 ? 2 : dtype == ORC_FP8 ? 1 : 4; }
static int factor_dtype(int dtype) { return dtype == ORC_FP8 ? ORC_BF16 : dtype; }

/* Stored element -> double; an fp8 code gives its code value (the caller scales). */
static double load_elem(int dtype, const void* base, int64_t i) {
    if (dtype == ORC_BF16) return orc_bf16_to_double(((const uint16_t*)base)[i]);
    if (dtype == ORC_FP8) return orc_fp8_to_double(((const uint8_t*)base)[i]);
    return (double)((const float*)base)[i];
}

/* y (for fp8: already divided by the scale) -> stored element. */
static void store_elem(int dtype, void* base, int64_t i, double y) {
    if (dtype == ORC_BF16) ((uint16_t*)base)[i] = orc_bf16_from_double(y);
    else if (dtype == ORC_FP8) ((uint8_t*)base)[i] = orc_fp8_from_double(y);
    else ((float*)base)[i] = (float)y; /* C conversion: round to nearest even */
}

static void copy_elem(int dtype, void* dst, int64_t i, const void* src, int64_t k) {
    int es = elem_size(dtype);
    memcpy((char*)dst + i * es, (const char*)src + k * es, (size_t)es);
}

/* ------------------------------------------------------------- relocation */

/* Angular frequency of rotary pair i in a head that rotates r dims:
 * theta^(-2i/r) (reading: the pages name RoPE but print no formula). */
double orc_freq(double theta, int r, int i) {
    return pow(theta, -2.0 * (double)i / (double)r);
}

/* Positional variant of the rotation: pairing and M-RoPE sections. */
typedef struct {
    int32_t pairing;          /* 0: NeoX half-split (i, i + r/2); 1: interleaved (2i, 2i + 1) */
    int32_t num_sections;     /* 0 or 1: one delta per chunk; 2..4: M-RoPE sections */
    int32_t section_pairs[4]; /* pairs per section, in pair order; they sum to r/2 */
} orc_rope;

static int rope_sections(const orc_rope* q) {
    return (q && q->num_sections > 1) ? q->num_sections : 1;
}

/* Section of rotary pair i. */
static int section_of(const orc_rope* q, int i) {
    int S = rope_sections(q), end = 0;
    for (int s = 0; s < S; ++s) {
        end += (S == 1) ? (1 << 30) : q->section_pairs[s];
        if (i < end) return s;
    }
    return S - 1;
}

/* Dims of rotary pair i in a head that rotates r dims. */
static void pair_dims(const orc_rope* q, int r, int i, int* d0, int* d1) {
    if (q && q->pairing == 1) { *d0 = 2 * i; *d1 = 2 * i + 1; }
    else { *d0 = i; *d1 = i + r / 2; }
}

/* Rotary pair that dim d (< r) belongs to. */
static int pair_of_dim(const orc_rope* q, int r, int d) {
    if (q && q->pairing == 1) return d / 2;
    return d < r / 2 ? d : d - r / 2;
}

/* Whether dim d of a head moves under the per-section deltas. */
static int dim_moves(const orc_rope* q, int r, int d, const int64_t* delta) {
    if (d >= r) return 0;
    return delta[section_of(q, pair_of_dim(q, r, d))] != 0;
}

/* y = R(delta) x for one head of `dim` values, in fp64 ([K §2, "Relocacao"]), with
 * the pairing and sections of `q` (NULL: NeoX, one section).  delta holds one value
 * per section.  Pairs whose section delta is 0 and dims >= r are copied. */
void orc_rotate_head_spec_f64(const double* x, double* y, int dim, int r, double theta,
                              const int64_t* delta, const orc_rope* q) {
    for (int d = 0; d < dim; ++d) y[d] = x[d];
    if (r == 0) return;
    int half = r / 2;
    for (int i = 0; i < half; ++i) {
        int64_t dl = delta[section_of(q, i)];
        if (dl == 0) continue;
        int d0, d1;
        pair_dims(q, r, i, &d0, &d1);
        double phi = (double)dl * orc_freq(theta, r, i);
        double cs = cos(phi), sn = sin(phi);
        double a = x[d0], b = x[d1];
        y[d0] = a * cs - b * sn;
        y[d1] = b * cs + a * sn;
    }
}

/* The plain form: NeoX pairing, one delta.  Dim i < r/2 pairs with dim i + r/2. */
void orc_rotate_head_f64(const double* x, double* y, int dim, int r,
                         double theta, int64_t delta) {
    orc_rotate_head_spec_f64(x, y, dim, r, theta, &delta, NULL);
}

/* y[f] += sum_k u[k] * V[f][k] for f < F: one token row of U_m V_m^T
 * ([K §2, reuse equation and "Aplicacao de Patch"]). V is [F][m]. */
void orc_patch_row_f64(double* y, int F, int m, const double* u, const double* V) {
    for (int f = 0; f < F; ++f) {
        double s = 0.0;
        for (int k = 0; k < m; ++k) s += u[k] * V[(int64_t)f * m + k];
        y[f] += s;
    }
}

/* One token row of one channel (heads x dim values, head-major), in fp64:
 * rotate every head, then add the patch row (m may be 0). */
void orc_row_spec_f64(const double* x, double* y, int heads, int dim, int r, double theta,
                      const int64_t* delta, const orc_rope* q, int m, const double* u,
                      const double* V) {
    for (int h = 0; h < heads; ++h)
        orc_rotate_head_spec_f64(x + (int64_t)h * dim, y + (int64_t)h * dim, dim, r, theta,
                                 delta, q);
    if (m > 0) orc_patch_row_f64(y, heads * dim, m, u, V);
}

void orc_row_f64(const double* x, double* y, int heads, int dim, int r, double theta,
                 int64_t delta, int m, const double* u, const double* V) {
    orc_row_spec_f64(x, y, heads, dim, r, theta, &delta, NULL, m, u, V);
}

/* One token row in storage format (dtype 0 = bf16 bits, 1 = fp32, 2 = fp8 E4M3
 * codes with dequantisation scale `scale`): x_in and out hold heads*dim contiguous
 * elements, u holds m, V holds [heads*dim][m], in the dtype's factor type (bf16 for
 * fp8, else the dtype).  out may equal x_in.  The row's values are scale * x (scale
 * is 1 but for fp8); the result is divided by the scale before it is stored.  With
 * m = 0, every element the rotation does not move keeps its bits. Returns 0, or -1
 * on bad arguments. */
int orc_row_spec_scaled(int dtype, double scale, const void* x_in, void* out, int heads,
                        int dim, int r, double theta, const int64_t* delta, const orc_rope* q,
                        int m, const void* u, const void* V) {
    if ((dtype != ORC_BF16 && dtype != ORC_F32 && dtype != ORC_FP8) || heads < 1 || dim < 1 ||
        r < 0 || r > dim || (r & 1) || m < 0 || !(scale > 0) || !isfinite(scale))
        return -1;
    if (q && q->num_sections > 1) {
        int sum = 0;
        if (q->num_sections > 4) return -1;
        for (int k = 0; k < q->num_sections; ++k) {
            if (q->section_pairs[k] < 0) return -1;
            sum += q->section_pairs[k];
        }
        if (r > 0 && sum != r / 2) return -1;
    }
    int64_t F = (int64_t)heads * dim;
    double* x = (double*)malloc(sizeof(double) * F);
    double* y = (double*)malloc(sizeof(double) * F);
    double* ud = (double*)malloc(sizeof(double) * (m > 0 ? m : 1));
    double* vd = (double*)malloc(sizeof(double) * (m > 0 ? F * m : 1));
    if (!x || !y || !ud || !vd) { free(x); free(y); free(ud); free(vd); return -1; }
    for (int64_t f = 0; f < F; ++f) x[f] = scale * load_elem(dtype, x_in, f);
    for (int k = 0; k < m; ++k) ud[k] = load_elem(factor_dtype(dtype), u, k);
    for (int64_t i = 0; i < F * m; ++i) vd[i] = load_elem(factor_dtype(dtype), V, i);
    orc_row_spec_f64(x, y, heads, dim, r, theta, delta, q, m, ud, vd);
    for (int64_t f = 0; f < F; ++f) {
        int d = (int)(f % dim);
        int moved = m > 0 || dim_moves(q, r, d, delta);
        if (moved) store_elem(dtype, out, f, y[f] / scale);
        else if (out != x_in) copy_elem(dtype, out, f, x_in, f);
    }
    free(x); free(y); free(ud); free(vd);
    return 0;
}

int orc_row_spec(int dtype, const void* x_in, void* out, int heads, int dim, int r,
                 double theta, const int64_t* delta, const orc_rope* q, int m, const void* u,
                 const void* V) {
    return orc_row_spec_scaled(dtype, 1.0, x_in, out, heads, dim, r, theta, delta, q, m, u, V);
}

int orc_row(int dtype, const void* x_in, void* out, int heads, int dim, int r,
            double theta, int64_t delta, int m, const void* u, const void* V) {
    return orc_row_spec(dtype, x_in, out, heads, dim, r, theta, &delta, NULL, m, u, V);
}

/* ---------------------------------------------------------- whole operator */

typedef struct {
    void* data;               /* element (layer 0, slot 0, head 0, dim 0) */
    int32_t heads, dim, rope_dim;
    int32_t pad_;
    int64_t layer_stride, slot_stride, head_stride, page_stride; /* elements */
    const void* U;            /* [layers][total_tokens][m] or NULL when m = 0 */
    const void* V;            /* [layers][chunks][heads*dim][m] or NULL */
    const float* scale;       /* fp8: [layers] dequantisation scales; else unused */
} orc_channel;

typedef struct {
    int32_t dtype, num_layers, num_channels, page_size;
    orc_channel ch[2];
    double theta;
    const int32_t* block_table; /* [ceil(total_tokens / page_size)] when paged */
    int64_t total_tokens;
    const int64_t* offsets;     /* [num_chunks + 1], 0 = o_0 <= ... = total */
    const int64_t* delta;       /* [num_chunks][sections] (sections = 1 without M-RoPE) */
    int32_t num_chunks, rank;
    orc_rope rope;              /* pairing and M-RoPE sections */
} orc_problem;

/* Element offset of (layer, logical token t, head h, dim 0).  Contiguous: the
 * slot is the token.  Paged with page size P: the logical page t / P is looked
 * up in the block table and t mod P is the slot inside that pool page. */
int64_t orc_row_offset(const orc_channel* c, int32_t page_size, const int32_t* bt,
                       int64_t layer, int64_t t, int64_t h) {
    int64_t slot;
    if (page_size > 0)
        slot = (int64_t)bt[t / page_size] * c->page_stride + (t % page_size) * c->slot_stride;
    else
        slot = t * c->slot_stride;
    return layer * c->layer_stride + slot + h * c->head_stride;
}

static int64_t chunk_of(const orc_problem* p, int64_t t) {
    for (int32_t j = 0; j < p->num_chunks; ++j)
        if (t >= p->offsets[j] && t < p->offsets[j + 1]) return j;
    return -1;
}

/* Sum of the magnitudes of the terms that make each fp64 row value: for a rotated
 * pair |a cos| + |b sin| (and |b cos| + |a sin|), |x| for an unrotated dim, plus
 * sum_k |u_k V[f][k]| for the patch.  It bounds the fp32 evaluation error of any
 * ordering of the same terms; the parity tolerance near cancellation scales with it. */
void orc_row_magnitude_spec_f64(const double* x, double* s, int heads, int dim, int r,
                                double theta, const int64_t* delta, const orc_rope* q, int m,
                                const double* u, const double* V) {
    int half = r / 2;
    for (int h = 0; h < heads; ++h) {
        const double* xh = x + (int64_t)h * dim;
        double* sh = s + (int64_t)h * dim;
        for (int d = 0; d < dim; ++d) sh[d] = fabs(xh[d]);
        for (int i = 0; i < half; ++i) {
            int64_t dl = delta[section_of(q, i)];
            if (dl == 0) continue;
            int d0, d1;
            pair_dims(q, r, i, &d0, &d1);
            double phi = (double)dl * orc_freq(theta, r, i);
            double cs = fabs(cos(phi)), sn = fabs(sin(phi));
            double a = fabs(xh[d0]), b = fabs(xh[d1]);
            sh[d0] = a * cs + b * sn;
            sh[d1] = b * cs + a * sn;
        }
    }
    int64_t F = (int64_t)heads * dim;
    for (int64_t f = 0; f < F; ++f)
        for (int k = 0; k < m; ++k) s[f] += fabs(u[k] * V[f * m + k]);
}

void orc_row_magnitude_f64(const double* x, double* s, int heads, int dim, int r,
                           double theta, int64_t delta, int m, const double* u,
                           const double* V) {
    orc_row_magnitude_spec_f64(x, s, heads, dim, r, theta, &delta, NULL, m, u, V);
}

/* The reuse operator over a whole problem, in place on host memory.  When y_out[c]
 * (and s_out[c]) are given, they are fp64 arrays laid out exactly like channel c's
 * elements (same offsets from the channel's data pointer); every element the call
 * computes gets its unrounded value there (and its magnitude bound), every other
 * element is left as the caller filled it.  With fp8 codes both are divided by the
 * layer's scale (code units, the grid the result is rounded on).  Returns 0, or -1
 * on bad arguments. */
int orc_relocate_patch_ex(const orc_problem* p, double* const* y_out, double* const* s_out) {
    if (!p || p->num_channels < 1 || p->num_channels > 2 || p->rank < 0 ||
        (p->dtype != ORC_BF16 && p->dtype != ORC_F32 && p->dtype != ORC_FP8))
        return -1;
    int64_t T = p->total_tokens, L = p->num_layers;
    if (T == 0 || L == 0 || p->num_chunks == 0) return 0;
    int es = elem_size(p->dtype), fs = elem_size(factor_dtype(p->dtype));
    int m = p->rank;
    int bad = 0;
    for (int c = 0; c < p->num_channels; ++c) {
        const orc_channel* ch = &p->ch[c];
        int64_t F = (int64_t)ch->heads * ch->dim;
        double* yo = y_out ? y_out[c] : NULL;
        double* so = s_out ? s_out[c] : NULL;
        if (m == 0 && ch->rope_dim == 0) continue; /* never read nor written */
#pragma omp parallel for collapse(2) schedule(dynamic, 64) reduction(|:bad)
        for (int64_t l = 0; l < L; ++l) {
            for (int64_t t = 0; t < T; ++t) {
                int64_t j = chunk_of(p, t);
                if (j < 0) { bad = 1; continue; }
                const int64_t* dj = p->delta + j * rope_sections(&p->rope);
                int any = 0;
                for (int k = 0; k < rope_sections(&p->rope); ++k) any |= dj[k] != 0;
                if (m == 0 && !any) continue;
                char* row = (char*)malloc((size_t)(F * es));
                double* x = (double*)malloc(sizeof(double) * F);
                double* y = (double*)malloc(sizeof(double) * F);
                double* s = (double*)malloc(sizeof(double) * F);
                double* ud = (double*)malloc(sizeof(double) * (m > 0 ? m : 1));
                double* vd = (double*)malloc(sizeof(double) * (m > 0 ? F * m : 1));
                int64_t* offs = (int64_t*)malloc(sizeof(int64_t) * ch->heads);
                for (int64_t h = 0; h < ch->heads; ++h) {
                    offs[h] = orc_row_offset(ch, p->page_size, p->block_table, l, t, h);
                    memcpy(row + h * ch->dim * es, (char*)ch->data + offs[h] * es, (size_t)ch->dim * es);
                }
                const void* u = NULL;
                const void* V = NULL;
                double sc = p->dtype == ORC_FP8 ? (double)ch->scale[l] : 1.0;
                if (m > 0) {
                    u = (const char*)ch->U + ((l * T + t) * m) * fs;
                    V = (const char*)ch->V + ((l * p->num_chunks + j) * F * m) * fs;
                    for (int k = 0; k < m; ++k) ud[k] = load_elem(factor_dtype(p->dtype), u, k);
                    for (int64_t i = 0; i < F * m; ++i)
                        vd[i] = load_elem(factor_dtype(p->dtype), V, i);
                }
                if (yo) {
                    for (int64_t f = 0; f < F; ++f) x[f] = sc * load_elem(p->dtype, row, f);
                    orc_row_spec_f64(x, y, ch->heads, ch->dim, ch->rope_dim, p->theta, dj, &p->rope,
                                     m, ud, vd);
                    orc_row_magnitude_spec_f64(x, s, ch->heads, ch->dim, ch->rope_dim, p->theta, dj,
                                               &p->rope, m, ud, vd);
                }
                if (orc_row_spec_scaled(p->dtype, sc, row, row, ch->heads, ch->dim, ch->rope_dim,
                                        p->theta, dj, &p->rope, m, u, V) != 0)
                    bad = 1;
                for (int64_t h = 0; h < ch->heads; ++h) {
                    memcpy((char*)ch->data + offs[h] * es, row + h * ch->dim * es, (size_t)ch->dim * es);
                    if (yo) {
                        for (int d = 0; d < ch->dim; ++d) {
                            int moved = m > 0 || dim_moves(&p->rope, ch->rope_dim, d, dj);
                            if (!moved) continue;
                            yo[offs[h] + d] = y[h * ch->dim + d] / sc;
                            if (so) so[offs[h] + d] = s[h * ch->dim + d] / sc;
                        }
                    }
                }
                free(row); free(x); free(y); free(s); free(ud); free(vd); free(offs);
            }
        }
    }
    return bad ? -1 : 0;
}

int orc_relocate_patch(const orc_problem* p) { return orc_relocate_patch_ex(p, NULL, NULL); }

/* Recall, the reversible eviction of [K §3, the three cheap window operations]: an
 * evicted chunk is rebuilt from its canonical store with a patch for its new context.
 * Out of place: each row is read from `src` (its layout, block table, chunks, deltas,
 * factors and rank) and the whole result row goes to the same token of `dst`, of
 * which only the channel data pointers, strides, page size and block table are read.
 * Every element of the row is written; elements that neither the rotation nor the
 * patch changes are copied bit for bit, so a chunk with delta 0 and no patch is a
 * plain copy.  src is never written.  With fp8 codes the destination keeps the
 * source's scales (its own are not read).  y_out / s_out are laid out like dst; the
 * computed elements get their fp64 value and magnitude bound there (fp8: divided by
 * the scale, in code units).  Returns 0, or -1 on bad arguments. */
int orc_recall_patch_ex(const orc_problem* src, const orc_problem* dst, double* const* y_out,
                        double* const* s_out) {
    if (!src || !dst || src->num_channels < 1 || src->num_channels > 2 || src->rank < 0 ||
        (src->dtype != ORC_BF16 && src->dtype != ORC_F32 && src->dtype != ORC_FP8) ||
        dst->dtype != src->dtype ||
        dst->num_channels != src->num_channels || dst->num_layers != src->num_layers)
        return -1;
    for (int c = 0; c < src->num_channels; ++c)
        if (dst->ch[c].heads != src->ch[c].heads || dst->ch[c].dim != src->ch[c].dim)
            return -1;
    int64_t T = src->total_tokens, L = src->num_layers;
    if (T == 0 || L == 0 || src->num_chunks == 0) return 0;
    int es = elem_size(src->dtype), fs = elem_size(factor_dtype(src->dtype));
    int m = src->rank;
    int bad = 0;
    for (int c = 0; c < src->num_channels; ++c) {
        const orc_channel* sc = &src->ch[c];
        const orc_channel* dc = &dst->ch[c];
        int64_t F = (int64_t)sc->heads * sc->dim;
        double* yo = y_out ? y_out[c] : NULL;
        double* so = s_out ? s_out[c] : NULL;
#pragma omp parallel for collapse(2) schedule(dynamic, 64) reduction(|:bad)
        for (int64_t l = 0; l < L; ++l) {
            for (int64_t t = 0; t < T; ++t) {
                int64_t j = chunk_of(src, t);
                if (j < 0) { bad = 1; continue; }
                const int64_t* dj = src->delta + j * rope_sections(&src->rope);
                char* row = (char*)malloc((size_t)(F * es));
                char* out = (char*)malloc((size_t)(F * es));
                double* x = (double*)malloc(sizeof(double) * F);
                double* y = (double*)malloc(sizeof(double) * F);
                double* s = (double*)malloc(sizeof(double) * F);
                double* ud = (double*)malloc(sizeof(double) * (m > 0 ? m : 1));
                double* vd = (double*)malloc(sizeof(double) * (m > 0 ? F * m : 1));
                for (int64_t h = 0; h < sc->heads; ++h) {
                    int64_t o = orc_row_offset(sc, src->page_size, src->block_table, l, t, h);
                    memcpy(row + h * sc->dim * es, (const char*)sc->data + o * es, (size_t)sc->dim * es);
                }
                const void* u = NULL;
                const void* V = NULL;
                double qs = src->dtype == ORC_FP8 ? (double)sc->scale[l] : 1.0;
                if (m > 0) {
                    u = (const char*)sc->U + ((l * T + t) * m) * fs;
                    V = (const char*)sc->V + ((l * src->num_chunks + j) * F * m) * fs;
                    for (int k = 0; k < m; ++k) ud[k] = load_elem(factor_dtype(src->dtype), u, k);
                    for (int64_t i = 0; i < F * m; ++i)
                        vd[i] = load_elem(factor_dtype(src->dtype), V, i);
                }
                if (yo) {
                    for (int64_t f = 0; f < F; ++f) x[f] = qs * load_elem(src->dtype, row, f);
                    orc_row_spec_f64(x, y, sc->heads, sc->dim, sc->rope_dim, src->theta, dj,
                                     &src->rope, m, ud, vd);
                    orc_row_magnitude_spec_f64(x, s, sc->heads, sc->dim, sc->rope_dim, src->theta,
                                               dj, &src->rope, m, ud, vd);
                }
                if (orc_row_spec_scaled(src->dtype, qs, row, out, sc->heads, sc->dim, sc->rope_dim,
                                        src->theta, dj, &src->rope, m, u, V) != 0)
                    bad = 1;
                for (int64_t h = 0; h < sc->heads; ++h) {
                    int64_t o = orc_row_offset(dc, dst->page_size, dst->block_table, l, t, h);
                    memcpy((char*)dc->data + o * es, out + h * sc->dim * es, (size_t)sc->dim * es);
                    if (yo) {
                        for (int d = 0; d < sc->dim; ++d) {
                            int moved = m > 0 || dim_moves(&src->rope, sc->rope_dim, d, dj);
                            if (!moved) continue;
                            yo[o + d] = y[h * sc->dim + d] / qs;
                            if (so) so[o + d] = s[h * sc->dim + d] / qs;
                        }
                    }
                }
                free(row); free(out); free(x); free(y); free(s); free(ud); free(vd);
            }
        }
    }
    return bad ? -1 : 0;
}

/* Relocate-on-read decode attention, the use of the rebuilt cache that [K §3]
 * describes as a hook in front of the attention kernel: the relocated and patched
 * keys and values are consumed by attention instead of being written back.  For
 * layer l and query head h (its KV head is g = h / (Hq / Hkv), grouped-query
 * attention), over every token t of every chunk j whose slot exists:
 *     K'_t = R(delta_j) K_t + U_K[l][t] V_K[l][j]^T    (head g's features)
 *     V'_t = V_t           + U_V[l][t] V_V[l][j]^T
 *     s_t  = scale * q[l][h] . K'_t
 *     out[l][h] = sum_t softmax(s)_t V'_t,   lse[l][h] = log sum_t exp(s_t)
 * K' and V' are the operator's values before rounding (the row function's fp64
 * result): the attention reads them, nothing stores them.  Channel 0 is K and
 * channel 1 is V, with equal heads and dim.  q and out are [L][Hq][dim] fp64, lse is
 * [L][Hq] (may be NULL).  A head with no token gets out = 0 and lse = -inf.  mag
 * (may be NULL, [L][Hq][dim]) receives sum_t softmax(s)_t |V'_t|, the scale of the
 * output's rounding error used by the parity tolerance.  Returns 0, or -1 on bad
 * arguments. */
int orc_attend(const orc_problem* p, int num_q_heads, double scale, const double* q,
               double* out, double* lse, double* mag) {
    if (!p || p->num_channels != 2 || p->rank < 0 || num_q_heads < 1 ||
        (p->dtype != ORC_BF16 && p->dtype != ORC_F32 && p->dtype != ORC_FP8))
        return -1;
    const orc_channel* kc = &p->ch[0];
    const orc_channel* vc = &p->ch[1];
    if (kc->heads != vc->heads || kc->dim != vc->dim || num_q_heads % kc->heads) return -1;
    int64_t T = p->total_tokens, L = p->num_layers;
    int H = kc->heads, D = kc->dim, G = num_q_heads / H, m = p->rank;
    int64_t F = (int64_t)H * D;
    int fs = elem_size(factor_dtype(p->dtype));
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t l = 0; l < L; ++l) {
        double* kp = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * F);
        double* vp = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * F);
        char* ok = (char*)calloc((size_t)(T > 0 ? T : 1), 1);
        double* x = (double*)malloc(sizeof(double) * F);
        double* ud = (double*)malloc(sizeof(double) * (m > 0 ? m : 1));
        double* vd = (double*)malloc(sizeof(double) * (m > 0 ? F * m : 1));
        double* sc = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        /* the relocated rows, in fp64, of both channels */
        for (int64_t t = 0; t < T; ++t) {
            int64_t j = chunk_of(p, t);
            if (j < 0) { bad = 1; continue; }
            if (p->page_size > 0) {
                int64_t pg = p->block_table[t / p->page_size];
                if (pg < 0) continue; /* no slot: the token is not attended */
            }
            ok[t] = 1;
            const int64_t* dj = p->delta + j * rope_sections(&p->rope);
            for (int c = 0; c < 2; ++c) {
                const orc_channel* ch = &p->ch[c];
                double sl = p->dtype == ORC_FP8 ? (double)ch->scale[l] : 1.0;
                for (int64_t h = 0; h < H; ++h) {
                    int64_t o = orc_row_offset(ch, p->page_size, p->block_table, l, t, h);
                    for (int d = 0; d < D; ++d) x[h * D + d] = sl * load_elem(p->dtype, ch->data, o + d);
                }
                if (m > 0) {
                    const char* u = (const char*)ch->U + ((l * T + t) * m) * fs;
                    const char* V = (const char*)ch->V + ((l * p->num_chunks + j) * F * m) * fs;
                    for (int k = 0; k < m; ++k) ud[k] = load_elem(factor_dtype(p->dtype), u, k);
                    for (int64_t i = 0; i < F * m; ++i)
                        vd[i] = load_elem(factor_dtype(p->dtype), V, i);
                }
                orc_row_spec_f64(x, (c == 0 ? kp : vp) + t * F, H, D, ch->rope_dim, p->theta, dj,
                                 &p->rope, m, ud, vd);
            }
        }
        /* attention of every query head */
        for (int hq = 0; hq < num_q_heads; ++hq) {
            int g = hq / G;
            const double* qh = q + (l * num_q_heads + hq) * D;
            double mx = -INFINITY;
            for (int64_t t = 0; t < T; ++t) {
                if (!ok[t]) continue;
                double s = 0.0;
                for (int d = 0; d < D; ++d) s += qh[d] * kp[t * F + g * D + d];
                sc[t] = scale * s;
                if (sc[t] > mx) mx = sc[t];
            }
            double* oh = out + (l * num_q_heads + hq) * D;
            double* mh = mag ? mag + (l * num_q_heads + hq) * D : NULL;
            for (int d = 0; d < D; ++d) oh[d] = 0.0;
            if (mh) for (int d = 0; d < D; ++d) mh[d] = 0.0;
            double sum = 0.0;
            if (mx > -INFINITY) {
                for (int64_t t = 0; t < T; ++t) {
                    if (!ok[t]) continue;
                    double w = exp(sc[t] - mx);
                    sum += w;
                    for (int d = 0; d < D; ++d) oh[d] += w * vp[t * F + g * D + d];
                    if (mh) for (int d = 0; d < D; ++d) mh[d] += w * fabs(vp[t * F + g * D + d]);
                }
                for (int d = 0; d < D; ++d) oh[d] /= sum;
                if (mh) for (int d = 0; d < D; ++d) mh[d] /= sum;
            }
            if (lse) lse[l * num_q_heads + hq] = mx > -INFINITY ? mx + log(sum) : -INFINITY;
        }
        free(kp); free(vp); free(ok); free(x); free(ud); free(vd); free(sc);
    }
    return bad ? -1 : 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Host threads the OpenMP loops use from now on (n >= 1); the arithmetic and its order
 * per element do not depend on it. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_struct_sizes(int which) {
    return which == 0 ? (int)sizeof(orc_channel) : (int)sizeof(orc_problem);
}
