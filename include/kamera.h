/*
 * kamera.h: C ABI of the Kamera relocate + patch operator on AMD Instinct MI355X (gfx950).
 *
 * The operator rebuilds a reused KV chunk at a new position
 * ("Kamera: KV Cache Multimodal Unificado e Invariante a Posicao para Reuso sem
 * Treinamento", gist.science/pt/paper/2606.23581, §2, reuse equation):
 *
 *     KV(B|A)  ~=  R(delta) * KV(B|empty)  +  U_m V_m^T
 *
 *   - R(delta): the cached keys, stored rotated at their old positions, are turned
 *     by the RoPE phase shift delta = new position - old position (same page, §2,
 *     "Relocacao": an exact rotation, no network pass).  Values and the MLA latent
 *     c_KV have no position and are not rotated (same page, §2, architecture list;
 *     and "Modelos Tomam Notas no Prefill", gist.science/pt/paper/2606.17107, §3B:
 *     keys are re-rotated, values are carried over unchanged).
 *   - U_m V_m^T: a rank-m conditioning patch, token factor U_m [T, m] and feature
 *     factor V_m [F, m], added to every patched channel (same Kamera page, §2,
 *     "Aplicacao de Patch"; MLA patches both of its channels, §2 architecture list).
 *   - With m = 0 the call is the rotation-only path that serves sliding-window
 *     survival (same page, §3, "Sobrevivencia de Janela Deslizante").
 *
 * Readings fixed by this library where the pages print no formula:
 *   - NeoX half-split pairing: in a head whose first rope_dim dims rotate, rotary
 *     pair i (i < rope_dim/2) is dims (i, i + rope_dim/2); it turns by angle
 *     delta * theta^(-2i/rope_dim); (a, b) -> (a cos - b sin, b cos + a sin).  Dims >=
 *     rope_dim do not rotate.  KAMERA_INTERLEAVED pairs dims (2i, 2i + 1) instead.
 *   - M-RoPE ("Modelos Tomam Notas no Prefill", gist.science/pt/paper/2606.17107, §4:
 *     image KV is transplanted with M-RoPE re-rotation): positions are vectors of up
 *     to 4 components; the rotary pairs are cut, in pair order, into that many
 *     sections, and pair i of section s turns by delta[s] * theta^(-2i/rope_dim).  A
 *     pair whose section delta is 0 does not move.
 *   - The patch is added after the rotation; it is not rotated.
 *   - delta == 0 means R = identity exactly.
 *   - Each output element is rounded once to the storage type (round to nearest even).
 *     Angles are formed and reduced in fp64; the sums run in fp32.
 *   - 8-bit KV ("Modelos Tomam Notas no Prefill", closing summary: the method holds on
 *     FP8-quantised models): KAMERA_FP8_E4M3 elements are OCP FP8 E4M3 codes and each
 *     channel carries one dequantisation scale s per layer, value = s * code value.
 *     The operator acts on values and stores encode(result / s): the nearest code,
 *     ties to the even code, saturating at +-448 (NaN stays NaN).  The factors are
 *     bf16, in value units.
 *
 * Conventions for every entry point:
 *   - In place: the KV buffers named by the descriptor are read and overwritten
 *     (kamera_recall_patch alone writes a separate destination instead).
 *   - Ownership: the caller owns every buffer (KV, block table, chunk offsets,
 *     deltas, factors).  The library allocates no memory, keeps no per-call state
 *     and returns as soon as the work is enqueued on `stream` (stream order; no
 *     host synchronisation).  Work is safe to capture in a HIP graph.
 *   - Pointers marked "device" must be device-accessible (hipMalloc or torch CUDA
 *     tensors).  Descriptor structs themselves are host memory and are read only
 *     during the call.
 *   - Errors: every host-checkable argument error is reported before any HIP call
 *     is made, as a kamera_status; kamera_last_error() then holds a message for the
 *     calling thread.  A failed launch returns KAMERA_E_HIP.  Device-array
 *     preconditions (listed per field) are not checked; whatever their values, the
 *     kernels only address tokens in [0, total_tokens), chunks in [0, num_chunks)
 *     and pool pages in [0, num_pages).
 *   - Threading: reentrant; calls on different streams are independent.  Calls that
 *     touch the same KV elements must be ordered by the caller.
 */
#ifndef KAMERA_H
#define KAMERA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef KAMERA_API
#define KAMERA_API __attribute__((visibility("default")))
#endif

#define KAMERA_ABI_VERSION 5
#define KAMERA_MAX_RANK 256   /* largest patch rank m accepted */

typedef enum {
  KAMERA_OK = 0,
  KAMERA_E_NULL = 1,        /* a required pointer is NULL */
  KAMERA_E_SHAPE = 2,       /* a size, stride, rank or rope_dim is out of range */
  KAMERA_E_UNSUPPORTED = 3, /* dtype or pairing this library does not implement */
  KAMERA_E_ALIGN = 4,       /* a pointer is not aligned to its element size */
  KAMERA_E_ALIAS = 5,       /* factor memory overlaps KV memory, or a recall destination
                               overlaps its source or the factors */
  KAMERA_E_HIP = 6          /* the HIP runtime reported an error at launch */
} kamera_status;

typedef enum {
  KAMERA_BF16 = 0,
  KAMERA_F32 = 1,
  KAMERA_FP8_E4M3 = 2  /* OCP E4M3 codes (1 byte) with per-layer scales; bf16 factors */
} kamera_dtype;

typedef enum {
  KAMERA_NEOX_HALF = 0,   /* rotary pair i is dims (i, i + rope_dim/2) */
  KAMERA_INTERLEAVED = 1  /* rotary pair i is dims (2i, 2i + 1) */
} kamera_pairing;

#define KAMERA_MAX_SECTIONS 4  /* M-RoPE position components */

/* flags of kamera_kv_desc */
#define KAMERA_FLAG_GENERIC 1u /* run the plain per-row kernel instead of the tuned ones */

/* One cache channel: K or V (MHA/GQA); c_KV or k_rope (MLA).
 * Element (layer l, slot s, head h, dim d) sits at
 *     data + l*layer_stride + s*slot_stride + h*head_stride + d          (contiguous)
 *     data + l*layer_stride + p*page_stride + s*slot_stride + h*head_stride + d (paged:
 *           logical token t lives in pool page p = block_table[t / page_size],
 *           slot s = t mod page_size)
 * Strides are in elements and must be >= 0.  The element sets of distinct rows,
 * heads and channels must not overlap (precondition).  The MLA combined row
 * [c_KV(512) | k_rope(64)] is two channels over one buffer: data and data + 512,
 * slot_stride 576. */
typedef struct {
  void* data;          /* device; element (layer 0, slot 0, head 0, dim 0) */
  int32_t heads;       /* >= 1 */
  int32_t dim;         /* head dim D >= 1; feature width F = heads * dim */
  int32_t rope_dim;    /* even, 0 <= rope_dim <= dim; 0 = this channel never rotates */
  int32_t reserved0;   /* must be 0 */
  int64_t layer_stride, slot_stride, head_stride, page_stride;
  const float* scale;  /* KAMERA_FP8_E4M3: device [num_layers] dequantisation scales,
                          precondition finite and > 0; ignored for other dtypes */
} kamera_channel;

typedef struct {
  int32_t dtype;         /* kamera_dtype of the KV elements (and of the factors, which
                            are bf16 for KAMERA_FP8_E4M3) */
  int32_t num_layers;    /* >= 0 */
  int32_t num_channels;  /* 1 or 2 */
  int32_t pairing;       /* kamera_pairing */
  kamera_channel ch[2];  /* MHA/GQA: {K, V}; MLA: {c_KV, k_rope} */
  double rope_theta;     /* RoPE base, finite and > 0 when any rope_dim > 0 */
  int32_t page_size;     /* 0 = contiguous (slot = token); > 0 = paged */
  uint32_t flags;        /* KAMERA_FLAG_* */
  int64_t num_pages;     /* paged: pool pages per layer; block-table entries lie in [0, num_pages) */
  const int32_t* block_table; /* device [ceil(total_tokens / page_size)] when paged, else ignored.
                                 Precondition: entries pairwise distinct.  Tokens whose entry
                                 lies outside [0, num_pages) are left untouched. */
  int32_t num_sections;  /* 0 or 1: one delta per chunk; 2..KAMERA_MAX_SECTIONS: M-RoPE */
  int32_t section_pairs[KAMERA_MAX_SECTIONS]; /* M-RoPE: rotary pairs per section, in pair
                                 order, each >= 0, summing to rope_dim/2 of every channel
                                 with rope_dim > 0; entries past num_sections are ignored */
  int32_t reserved1;     /* must be 0 */
} kamera_kv_desc;

/* The chunks being moved.  Chunk j owns logical tokens [token_offsets[j], token_offsets[j+1]). */
typedef struct {
  int32_t num_chunks;      /* >= 0; 0 requires total_tokens == 0 */
  int32_t reserved0;       /* must be 0 */
  int64_t total_tokens;    /* host copy of token_offsets[num_chunks]; sizes the launch */
  const int64_t* token_offsets; /* device [num_chunks + 1]; precondition: 0 = o_0 <= o_1 <= ... = total_tokens */
  const int64_t* delta;    /* device [num_chunks][S], S = max(1, kv.num_sections): new position -
                              old position, one value per M-RoPE section; precondition
                              |delta| < 2^53 */
} kamera_chunks;

/* The rank-m patch, one factor pair per channel, in the KV dtype (bf16 for
 * KAMERA_FP8_E4M3), dense row-major:
 *   U[c]: [num_layers][total_tokens][rank]           token factor U_m, per layer
 *   V[c]: [num_layers][num_chunks][heads*dim][rank]  feature factor V_m, per layer and chunk
 * The same pointers may be passed for both channels when their shapes agree. */
typedef struct {
  int32_t rank;            /* 0 <= m <= KAMERA_MAX_RANK; 0 = no patch */
  int32_t reserved0;       /* must be 0 */
  const void* U[2];        /* device, read only; NULL allowed only when rank == 0 */
  const void* V[2];        /* device, read only; NULL allowed only when rank == 0 */
} kamera_patch;

/* Rotation only (m = 0).  Rotates dims [0, rope_dim) of every head of every channel
 * with rope_dim > 0, for every chunk with delta != 0.  Nothing else is written:
 * channels with rope_dim == 0 (V, c_KV), dims >= rope_dim, chunks with delta == 0 and
 * (M-RoPE) the pairs of sections whose delta is 0 keep their exact bits.  Kamera page
 * §3, sliding-window survival. */
KAMERA_API kamera_status kamera_relocate(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                              hipStream_t stream);

/* Relocate and patch: every element of every channel becomes
 * round(R(delta_j) x + sum_k U[c][l][t][k] * V[c][l][j][f][k]).  Kamera page §2,
 * reuse equation.  patch == NULL or patch->rank == 0 behaves as kamera_relocate. */
KAMERA_API kamera_status kamera_relocate_patch(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                                    const kamera_patch* patch, hipStream_t stream);

/* Relocate and patch with a caller workspace: the same operation and results as
 * kamera_relocate_patch (Kamera page §2, reuse equation), element for element; only the
 * order of the work differs.  When the call moves one chunk (num_chunks == 1) of a paged
 * cache whose page_size is a multiple of 16 and whose pool holds at most four times the
 * pages the chunk uses, the library first writes the inverse of the block table into
 * the workspace (pool page -> logical page; int32 per pool page) and then sweeps the
 * pool in page order, so that concurrent work touches neighbouring pool memory instead
 * of the table's scattered pages.  Other calls run exactly as kamera_relocate_patch and
 * leave the workspace alone.
 *   workspace: caller-owned device memory, 16-byte aligned, of at least the bytes
 *     kamera_relocate_workspace reports, or NULL (then the call is kamera_relocate_patch).
 *     Overwritten.  It must not overlap the cache, the factors, the block table, the
 *     offsets or the deltas (KAMERA_E_ALIAS); fewer bytes than needed: KAMERA_E_SHAPE.
 * Stream-ordered like every entry point: calls that share a workspace must be ordered. */
KAMERA_API kamera_status kamera_relocate_patch_ws(const kamera_kv_desc* kv,
                                       const kamera_chunks* chunks,
                                       const kamera_patch* patch, void* workspace,
                                       int64_t workspace_bytes, hipStream_t stream);

/* kamera_relocate_patch_ws for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * results, with the inverse block table held in a library-owned device array instead of
 * a caller workspace.  Nothing is allocated: the array (4 MiB, room for 1,048,576 pool
 * pages) is part of the library's device code, one copy per GPU, kept until the process
 * ends; the first call on a GPU looks its address up (a runtime query, no allocation).
 * A problem that would use more pool pages than that returns KAMERA_E_SHAPE before any
 * HIP call (kamera_relocate_patch_ws takes any size).  Every call on one GPU shares its
 * array: calls on that GPU that may overlap in time (different streams, no ordering)
 * race and must be ordered by the caller.  Problems that need no inverse table run as
 * kamera_relocate_patch.  Errors as for kamera_relocate_patch. */
KAMERA_API kamera_status kamera_relocate_patch_noalloc(const kamera_kv_desc* kv,
                                            const kamera_chunks* chunks,
                                            const kamera_patch* patch, hipStream_t stream);

/* Bytes of workspace kamera_relocate_patch_ws uses for this problem: 0 when it runs as
 * kamera_relocate_patch, else 4 bytes per pool page rounded up to 256.  Checks the
 * arguments as the call does (no HIP call). */
KAMERA_API kamera_status kamera_relocate_workspace(const kamera_kv_desc* kv,
                                        const kamera_chunks* chunks,
                                        const kamera_patch* patch, int64_t* bytes);

/* Recall, out of place: rebuild chunks from their canonical store into other cache
 * slots.  Kamera page §3, the three cheap window operations, recall (reversible
 * eviction): an evicted chunk is rehydrated from the canonical store with a patch for
 * its new context, without re-encoding it.
 *
 * Every row (layer l, token t, each head) of every channel is read through `src` and
 * the whole result row is written to the same (l, t) through `dst`:
 *     dst element = round(R(delta_j) x + sum_k U[c][l][t][k] * V[c][l][j][f][k])
 * Elements that neither the rotation nor the patch changes (rank 0 and rope_dim 0,
 * dims >= rope_dim, chunks with delta 0 at rank 0) are copied bit for bit.
 *   src: the canonical store (contiguous or paged); read only.  It is checked as the
 *        kv argument of kamera_relocate_patch is (factors overlapping it are rejected
 *        too).
 *   dst: the cache being filled.  dtype, num_layers, num_channels and each channel's
 *        heads, dim and rope_dim must equal src's; data, strides, page_size,
 *        num_pages and block_table are its own (destination tokens whose page id lies
 *        outside [0, num_pages) are skipped).  Its rope_theta, pairing, sections and
 *        (fp8) scales are not read: the source's apply, so an fp8 destination holds
 *        codes in the source's scales.
 *        Its memory must not overlap the source or the factors (KAMERA_E_ALIAS).
 *   patch == NULL or rank 0: rotation and copy only.
 * chunks, stream and errors as for kamera_relocate_patch. */
KAMERA_API kamera_status kamera_recall_patch(const kamera_kv_desc* src, const kamera_kv_desc* dst,
                                  const kamera_chunks* chunks, const kamera_patch* patch,
                                  hipStream_t stream);

/* ------------------------------------------------------------------ relocate-on-read attention
 *
 * Kamera page §3, production deployment: the rebuild runs as a hook in front of the
 * attention kernel.  This entry point is that use with nothing written back: decode
 * attention (one query per layer and query head) reads the cached keys and values and
 * consumes the relocated, patched ones directly,
 *     K'_t = R(delta_j) K_t + sum_k U[0][l][t][k] V[0][l][j][f][k]
 *     V'_t = V_t            + sum_k U[1][l][t][k] V[1][l][j][f][k]
 *     out[l][h] = sum_t softmax_t(scale * q[l][h] . K'_t) V'_t
 *     lse[l][h] = log sum_t exp(scale * q[l][h] . K'_t)
 * over every token t of every chunk j, query head h reading KV head
 * h / (num_q_heads / heads) (grouped-query attention).  K' and V' are the operator's
 * values before rounding; the cache is not modified.  The library evaluates the same
 * sums re-associated ((R(-delta) q) . K_t + (V_K^T q) . U[0][t], and V_V applied to
 * sum_t p_t U[1][t]), in fp32.
 *
 * kv: MHA/GQA, bf16 or fp8 E4M3 (values scale * code with each channel's per-layer
 *     scale, as for kamera_relocate_patch); channel 0 = K (its rope_dim, pairing and sections rotate),
 *     channel 1 = V (rope_dim 0); equal heads; dim 128; contiguous or paged (tokens
 *     whose block-table entry lies outside [0, num_pages) are not attended).  Row bases
 *     16-byte aligned (KAMERA_E_ALIGN: data 16-byte aligned, strides multiples of 8
 *     elements, of 16 for fp8), one layer of a
 *     channel spanning less than 2^31 - 64 bytes, total_tokens below 2^30, a block
 *     table below 2^29 entries.  Other shapes: KAMERA_E_UNSUPPORTED.
 * patch: NULL or rank 0 for plain attention; else a rank that is a multiple of 8, up
 *     to 128, with 16-byte aligned bf16 factors as for kamera_relocate_patch, one
 *     layer of U spanning less than 2^31 - 64 bytes.
 * A head with no attended token gets out = 0 and lse = -inf. */
typedef struct {
  int32_t num_q_heads;   /* Hq: a multiple of kv.heads, at most 8 times it */
  int32_t reserved0;     /* must be 0 */
  float scale;           /* softmax scale (for example dim^-1/2); finite */
  int32_t reserved1;     /* must be 0 */
  const float* q;        /* device [num_layers][num_q_heads][dim] fp32, read only: the query of
                            each layer, already rotated to its own position */
  float* out;            /* device [num_layers][num_q_heads][dim] fp32, written */
  float* lse;            /* device [num_layers][num_q_heads] fp32 (natural log), or NULL */
} kamera_attend_desc;

/* Bytes of workspace kamera_attend needs for this problem (0 when it is empty); the
 * prepared queries and the partial sums depend on the rank, so the patch is an input. */
KAMERA_API kamera_status kamera_attend_workspace(const kamera_kv_desc* kv,
                                      const kamera_chunks* chunks, const kamera_patch* patch,
                                      const kamera_attend_desc* attend, int64_t* bytes);

/* Stream-ordered.  workspace: caller-owned device memory of at least the bytes
 * kamera_attend_workspace reports, 16-byte aligned, overwritten.  out, lse and the
 * workspace must not overlap each other, q or the cache (KAMERA_E_ALIAS). */
KAMERA_API kamera_status kamera_attend(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                            const kamera_patch* patch, const kamera_attend_desc* attend,
                            void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ patch formation
 *
 * The step before the reuse operator: Kamera page §2, "Aplicacao de Patch" forms the
 * patch once, from one conditioned forward pass over [A, B] and an SVD that keeps the
 * top-m factors.  The forward pass is the caller's.  Given the deficit
 * Delta = KV(B|A) - KV(B|empty) of every layer and chunk of a channel, this writes
 * U_m = U[:, :m] diag(s[:m]) and V_m = V[:, :m] of each chunk's SVD Delta_j = U diag(s) V^T,
 * in the layouts kamera_patch takes, so U_m V_m^T is the best rank-m approximation of
 * Delta_j (Eckart-Young).  Singular vectors are unique only up to sign (and within
 * repeated singular values); their product is what the operator uses.
 *
 * Method: Gram matrix Delta_j^T Delta_j on MFMA (bf16 products, fp32 sums), subspace
 * iteration in fp32 with k = min(m + 16 rounded up to even, width, 128) columns,
 * Rayleigh-Ritz with a Jacobi eigensolver, U_m = Delta_j V_m.  Its error falls like
 * (lambda_{k+1} / lambda_i)^iterations for eigenvalue lambda_i = s_i^2; a chunk whose
 * singular values past m fall off is solved to fp32 precision in a few iterations.
 * Outputs are rounded to bf16 (sigma stays fp32). */
#define KAMERA_FORM_MAX_RANK 112

typedef struct {
  int32_t dtype;          /* KAMERA_BF16 (deficit and factors) */
  int32_t num_layers;     /* >= 0 */
  int32_t num_channels;   /* 1 or 2 */
  int32_t rank;           /* m, 1 <= m <= KAMERA_FORM_MAX_RANK */
  int32_t width[2];       /* F of each channel (heads * dim): a multiple of 64 in [64, 1024] */
  int32_t iterations;     /* subspace iterations after the first; 0 = 8; at most 64 */
  int32_t reserved0;      /* must be 0 */
  const void* delta[2];   /* device [num_layers][total_tokens][width] bf16, row-major, 16-byte
                             aligned; read only */
  void* U[2];             /* device out [num_layers][total_tokens][rank] bf16 */
  void* V[2];             /* device out [num_layers][num_chunks][width][rank] bf16 */
  float* sigma[2];        /* device out [num_layers][num_chunks][rank] fp32, or NULL */
} kamera_form_desc;

/* Bytes of workspace kamera_form_patch can use to hold up to 64 (layer, chunk)
 * problems at a time; any workspace of at least one problem's share works (in more
 * batches).  Checks the descriptor like kamera_form_patch. */
KAMERA_API kamera_status kamera_form_workspace(const kamera_form_desc* desc,
                                    const kamera_chunks* chunks, int64_t* bytes);

/* Forms the patch of every layer and chunk of every channel.  chunks: offsets and
 * total_tokens as for kamera_relocate_patch (its delta is not read).  The workspace is
 * caller-owned device memory, 256-byte aligned, overwritten; nothing else is
 * allocated.  The outputs must not overlap the deficit, each other or the workspace
 * (KAMERA_E_ALIAS).  Stream-ordered, like every entry point. */
KAMERA_API kamera_status kamera_form_patch(const kamera_form_desc* desc, const kamera_chunks* chunks,
                                void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* The first stage of kamera_form_patch on its own: the Gram matrix
 * G_j = Delta_j^T Delta_j (fp32 [width][width]) of every layer and chunk of every
 * channel, a dense contraction over the chunk's tokens on MFMA (bf16 products, fp32
 * sums).  G[c]: device out [num_layers][num_chunks][width][width] fp32, must not
 * overlap a deficit.  desc.rank, U, V, sigma and iterations are not read. */
KAMERA_API kamera_status kamera_form_gram(const kamera_form_desc* desc, const kamera_chunks* chunks,
                               float* const G[2], hipStream_t stream);

/* Orbit deficit: Kamera page §3, "Tres Operacoes de Janela Baratas", item 1
 * ("Reordenacao"): one patch averaged over permutations serves every order of a cached
 * set.  Given the deficit of a channel under each of num_orders orders of the set (each
 * in the chunks' canonical frames, laid out as kamera_form_desc.delta), this writes
 * their mean, out[i] = bf16(sum_p deltas[p * order_stride + i] / num_orders): the sum
 * in fp64 in order p = 0, 1, ..., one fp64 division, one rounding to nearest even.
 * kamera_form_patch on `out` then gives the orbit patch, the top-m factorization of the
 * mean deficit (among rank-m matrices it minimizes the squared error summed over the
 * orbit).
 *   deltas: device bf16, order p's deficit at element p * order_stride; read only.
 *   out: device bf16 [elements]; must not overlap any order's deficit (KAMERA_E_ALIAS).
 *   deltas and out 16-byte aligned, order_stride a multiple of 8 (KAMERA_E_ALIGN);
 *   1 <= num_orders <= 2^20, elements >= 0, order_stride >= elements (KAMERA_E_SHAPE).
 * A NaN input gives a NaN (sign unspecified); infinities follow fp64 arithmetic.
 * Stream-ordered; allocates nothing. */
KAMERA_API kamera_status kamera_orbit_mean(const void* deltas, int32_t num_orders, int64_t elements,
                                int64_t order_stride, void* out, hipStream_t stream);

/* Which kernels a call would launch, without launching anything (no HIP call).
 * Fills `out` and returns the status the call itself would return before launching. */
typedef struct {
  int32_t kernel[2];       /* per channel: 0 none, 1 rotate (tuned), 2 rotate+patch MFMA (tuned),
                              3 generic */
  int32_t launches;        /* kernel launches the call would make (the rotate+patch kernel
                              takes a second launch for the token groups that chunk
                              boundaries cut when boundaries outnumber token groups) */
  int32_t tokens_per_unit; /* tokens one workgroup of a tuned kernel covers */
  int64_t units;           /* workgroups of the tuned launches */
} kamera_plan_info;

KAMERA_API kamera_status kamera_plan(const kamera_kv_desc* kv, const kamera_chunks* chunks,
                          const kamera_patch* patch, kamera_plan_info* out);

/* Same for kamera_recall_patch (which launches every channel: each is written whole). */
KAMERA_API kamera_status kamera_recall_plan(const kamera_kv_desc* src, const kamera_kv_desc* dst,
                                 const kamera_chunks* chunks, const kamera_patch* patch,
                                 kamera_plan_info* out);

KAMERA_API const char* kamera_status_str(kamera_status s);
KAMERA_API const char* kamera_last_error(void); /* this thread's last failure message ("" if none) */
KAMERA_API int kamera_abi_version(void);        /* KAMERA_ABI_VERSION */

#ifdef __cplusplus
}
#endif
#endif /* KAMERA_H */
