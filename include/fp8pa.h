/*
 * fp8pa.h: paged flash-decode attention over an FP8 (OCP E4M3) KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one named by the solution record "How do I run paged
 * decode attention over an FP8 KV cache for a quantized MoE serving path,
 * with sliding windows, attention sinks and a custom scale?"
 * (cerinamroth.com, fields `title` and `summary`): decode-time attention of
 * new query tokens against a paged E4M3 key/value cache, with grouped KV
 * heads (`install.environment.special_requirements` of that record), an
 * optional sliding window, per-head attention-sink logits and a
 * caller-supplied softmax scale.  For every sequence b, query token i and
 * query head h, with g = h / (Hq / Hkv) and pos = seq_lens[b] - q_len + i:
 *
 *   K[t] = e4m3(k_cache[block_table[b][t / bt], t % bt, g, :]) * k_scale[g]
 *   V[t] = e4m3(v_cache[...same page and slot...]) * v_scale[g]
 *
 * (K scales may also come in k_groups groups along head_dim, the same
 * record's special requirements: element d of K[t] then takes
 * k_scale[g][d / (D / k_groups)]; V keeps one scale per head or tensor.)
 *   s_t  = sm_scale * dot(q[b, i, h, :], K[t])       for attended t
 *   out  = sum_t e^{s_t} V[t] / (sum_t e^{s_t} + e^{sinks[h]})
 *   lse  = ln(sum_t e^{s_t} + e^{sinks[h]})            (natural log)
 *
 * Attended keys: 0 <= t <= pos, and t >= pos - window + 1 when window > 0
 * (the last `window` positions, the query's own included).  The sink term
 * is absent when `sinks` is NULL.  A row with nothing to attend gets
 * out = 0 and lse = -inf (or the sink).  The cache writer multiplies by
 * 1 / k_scale before encoding (gist "Qwen3.8-27B ... on a single RTX 5090",
 * kernel `reshape_and_cache_nvfp4_kernel`), so codes decode to code * scale.
 *
 * Work is a split-KV partial pass plus a log-sum-exp merge of the splits, the
 * structure of FlashInfer PR #5591 (Summary: split producers and one LSE
 * reducer; workspace commit: caller-owned workspace carved into partial O
 * and partial LSE, no device allocation on any call path).
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller; they must
 *    stay valid until the work queued on `stream` has finished.  No call
 *    allocates, keeps per-call state or synchronises; the library holds a
 *    cache of each device's compute-unit count and, for
 *    fp8pa_decode_noalloc only, one fixed scratch array per device (a
 *    static device array, with its address looked up once per device).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is queued on it and the call returns at once; a call can be
 *    captured into a hipGraph from its first use.
 *  - Errors are reported as a status; nothing is printed, thrown or aborted.
 *    Host-checkable preconditions are checked before any work is queued.
 *    Device-resident values (seq_lens, block_table) are not checked, as that
 *    would need a synchronisation; see fp8pa_decode for their preconditions.
 */
#ifndef FP8PA_H_
#define FP8PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8pa_status {
  FP8PA_OK = 0,
  FP8PA_ERR_INVALID_ARG = 1,        /* a null required pointer, a bad size or count */
  FP8PA_ERR_UNSUPPORTED = 2,        /* a shape no kernel variant handles (e.g. head_dim 96) */
  FP8PA_ERR_WORKSPACE_TOO_SMALL = 3,
  FP8PA_ERR_MISALIGNED = 4,         /* a pointer breaks the documented alignment */
  FP8PA_ERR_HIP = 5                 /* the HIP runtime reported an error */
} fp8pa_status;

/* fp8pa_shape.flags bits, for testing and measurement; production calls pass 0. */
#define FP8PA_FLAG_FORCE_DOT  1 /* use the VALU dot-product kernel */
#define FP8PA_FLAG_FORCE_MFMA 2 /* use the FP8-MFMA kernel (needs block_tokens >= 16) */
#define FP8PA_FLAG_PARTIAL_ONLY 4 /* run the partial pass only: when the plan has a
                                     merge, it is not launched and out / lse are
                                     left unwritten (times the partial kernel) */

/* Byte layout of a KV page (fp8pa_shape.kv_layout, fp8pa_write_shape.kv_layout). */
#define FP8PA_LAYOUT_NHD 0 /* token-major: [num_blocks][bt][Hkv][D] */
#define FP8PA_LAYOUT_HND 1 /* head-major:  [num_blocks][Hkv][bt][D] (gist "Qwen3.8-27B ...
                              on a single RTX 5090", KV cache row and writer: a head's
                              tokens lie D bytes apart, heads bt * D apart) */

/* Element format of the KV pools (fp8pa_shape.kv_format, fp8pa_write_shape.kv_format). */
#define FP8PA_KV_E4M3  0 /* one OCP E4M3 byte per element: page = [bt][Hkv][D] or [Hkv][bt][D] */
#define FP8PA_KV_NVFP4 1 /* NVFP4 (gist "Qwen3.8-27B ... on a single RTX 5090", writer kernel
                            reshape_and_cache_nvfp4_kernel): each page is a data region of
                            4-bit E2M1 codes, two per byte (element 2i in the low nibble),
                            rows of D/2 bytes, followed by a scale region of one E4M3 byte per
                            16 elements, rows of D/16 bytes; rows are ordered by kv_layout.
                            A value reads as E2M1(code) * E4M3(block scale) * k_scale (v_scale). */
#define FP8PA_KV_MXFP8 2 /* MXFP8 (the fish-scales-ops README: 1 x 32 blocks sharing one
                            power-of-two UE8M0 scale): each page is a data region of E4M3
                            codes, rows of D bytes, followed by a scale region of one E8M0 byte
                            per 32 consecutive head_dim elements of a token, rows of D/32 bytes;
                            rows are ordered by kv_layout as for NVFP4.  A value reads as
                            E4M3(code) * 2^(s - 127) * k_scale (v_scale); s = 0xFF is NaN.
                            Supported scale bytes: 10 <= s <= 200.  Within them every element
                            is a normal bf16 number, so the kernels hold it exactly, and the
                            P.V sums stay finite (P <= 2^8 times elements below 2^82 over up
                            to 2^20 keys); the scores sm_scale * q.K stay finite as long as
                            the caller's queries keep them inside fp32's range.  Bytes 0..9
                            give elements below bf16's normal range, which the conversion may
                            flush, and 201..254 may overflow the fp32 sums: results over pages
                            holding such bytes are unspecified (the bytes live on the device
                            and are not checked). */

/* Host-known description of one decode call. */
typedef struct fp8pa_shape {
  int32_t batch;              /* B >= 1 sequences */
  int32_t q_len;              /* query tokens per sequence, >= 1 (q_len > 1: draft
                                 tokens, causal among themselves) */
  int32_t num_q_heads;        /* Hq >= 1 */
  int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;           /* D: 64, 128 or 256 */
  int32_t block_tokens;       /* bt: tokens per page, a power of two in [1, 1024] */
  int32_t num_blocks;         /* pages in each of the two pools, >= 1 */
  int32_t block_table_stride; /* elements between rows of block_table, >= 1 */
  int32_t max_seq_len;        /* an upper bound of every seq_lens[b], >= 1; sizes the
                                 split plan and the workspace */
  int32_t k_scale_count;      /* kg (per tensor) or Hkv * kg (per kv head, [Hkv][kg]),
                                 kg = max(k_groups, 1) */
  int32_t v_scale_count;      /* 1 or Hkv */
  int32_t k_groups;           /* 0 or 1: one K scale per head (or tensor); 2, 4, 8 or
                                 16: K scale groups along head_dim, D / k_groups >= 32,
                                 group j covering dims [j D / k_groups, (j+1) D / k_groups) */
  int32_t kv_layout;          /* FP8PA_LAYOUT_NHD (0) or FP8PA_LAYOUT_HND (1), both pools */
  int32_t kv_format;          /* FP8PA_KV_E4M3 (0), FP8PA_KV_NVFP4 (1) or FP8PA_KV_MXFP8 (2);
                                 the block-scaled formats need k_groups <= 1 */
  int32_t window;             /* <= 0: none; W > 0: the last W positions */
  float sm_scale;             /* softmax scale applied to q.K; finite */
  int32_t num_splits;         /* 0: the library plans; > 0 asks for that many KV
                                 splits at most (the MFMA kernel still splits so
                                 that no split spans more than 128 tiles) */
  int32_t flags;              /* FP8PA_FLAG_* bits, 0 in production */
  int64_t kv_page_stride;     /* bytes between consecutive pages of each pool; 0 = one page's
                                 own size (dense pools).  Larger strides let K and V pages
                                 interleave ([K page | V page] per block).  A multiple of 16;
                                 NVFP4 and MXFP8 pools whose own page size is not one need it
                                 (FP8PA_ERR_MISALIGNED otherwise). */
} fp8pa_shape;

/* How the keys of a sequence are divided among workgroups. */
#define FP8PA_SPLIT_DIRECT   0 /* one split; the partial kernel writes out/lse, no merge */
#define FP8PA_SPLIT_FIXED    1 /* every sequence: splits of tiles_per_split tiles */
#define FP8PA_SPLIT_BALANCED 2 /* the kernel reads all seq_lens and picks one chunk size
                                  (<= max_tiles_per_split) so that the (sequence, split)
                                  items of the whole batch come to about target_items,
                                  never more than the target_items + batch workgroup
                                  slots (the smaller chunk T / slots where it fits);
                                  idle workgroups exit */

/* The plan one call will run (see fp8pa_plan). */
typedef struct fp8pa_plan_info {
  int32_t variant;          /* 0 = VALU dot kernel, 1 = FP8-MFMA kernel */
  int32_t split_mode;       /* FP8PA_SPLIT_* */
  int32_t num_splits;       /* partial slots per query row: the most splits one
                               sequence can get */
  int32_t tiles_per_split;  /* 32-token tiles per split (BALANCED: the chunk floor,
                               64 keys per query row, kept while at least half of
                               target_items remain) */
  int32_t max_tiles_per_split; /* the largest chunk a split may take */
  int32_t target_items;     /* BALANCED: (sequence, split) items aimed at; else 0 */
  int32_t tile_tokens;      /* tokens per tile (32) */
  int32_t heads_per_wg;     /* kv heads per workgroup */
  int32_t waves_per_head;   /* wavefronts sharing one kv head's head_dim (1, or 2 at D = 256) */
  int32_t rows_per_group;   /* query rows (q heads x q tokens) per wavefront */
  int32_t row_groups;       /* ceil(Hq / Hkv * q_len / rows_per_group) */
  int32_t grid_wgs;         /* workgroups of the partial kernel */
  int32_t merge_launched;   /* 1 when num_splits > 1 and a merge kernel follows */
  int32_t heads_per_wave;   /* kv heads one wavefront takes (2 at head_dim 64 with
                               at most 8 query rows per kv head, else 1); a
                               workgroup has heads_per_wg / heads_per_wave *
                               waves_per_head wavefronts */
  int32_t row_blocks;       /* 16-row MFMA blocks one wavefront carries over the same
                               K/V registers (1, or 2 for more than 16 query
                               rows per kv head); rows_per_group = 16 * row_blocks */
  int32_t nontemporal_kv;   /* 1 when K/V loads bypass cache retention: each byte
                               is read by one wavefront (row_groups == 1) */
  int32_t row_groups_per_wg; /* row groups of one kv head whose wavefronts share each
                                K/V tile through LDS (4 or 8 with many query rows per
                                kv head); such a workgroup has that many wavefronts
                                and heads_per_wg = 1.  Otherwise 1. */
  uint64_t workspace_bytes; /* bytes fp8pa_decode needs in `workspace` */
  uint64_t workspace_lse_offset; /* byte offset of the partial LSE block in the
                                    workspace; the partial outputs start at 0.
                                    Both blocks use fp8pa_merge's layout
                                    ([B*q_len*Hq rows][num_splits](x head_dim)),
                                    followed by one word of plan state. */
} fp8pa_plan_info;

/*
 * fp8pa_plan: the plan fp8pa_decode would run for `shape` on a device with
 * `cu_count` compute units.  Pure host arithmetic; no GPU is touched.
 * Returns FP8PA_ERR_INVALID_ARG / FP8PA_ERR_UNSUPPORTED for shapes that
 * fp8pa_decode rejects.  The plan is a deterministic function of its
 * arguments, so a captured graph replays the same launches.
 */
fp8pa_status fp8pa_plan(const fp8pa_shape* shape, int32_t cu_count, fp8pa_plan_info* out);

/*
 * fp8pa_workspace_bytes: bytes of device workspace fp8pa_decode needs for
 * `shape` on HIP device `device` (its compute-unit count enters the plan).
 * 0 means no workspace.  Host only; queries the device attribute once.
 */
fp8pa_status fp8pa_workspace_bytes(const fp8pa_shape* shape, int device, size_t* bytes);

/*
 * fp8pa_decode: out[b, i, h, :] and lse[b, i, h] for every row, as defined at
 * the top of this file, on the current HIP device.
 *
 *   q            bf16  [B, q_len, Hq, D] contiguous
 *   k_cache      e4m3  [num_blocks, bt, Hkv, D] contiguous (token-major pages), or
 *                [num_blocks, Hkv, bt, D] with kv_layout = FP8PA_LAYOUT_HND
 *   v_cache      e4m3  the same shape and layout as k_cache
 *   block_table  int32 [B, block_table_stride]; entry j of row b is the page
 *                that holds tokens [j*bt, (j+1)*bt) of sequence b
 *   seq_lens     int32 [B]; tokens of each sequence, its q_len new ones included
 *   k_scale      float [k_scale_count], v_scale float [v_scale_count]
 *   sinks        float [Hq] or NULL
 *   out          bf16  [B, q_len, Hq, D] contiguous (written)
 *   lse          float [B, q_len, Hq] or NULL (written when not NULL)
 *   workspace    device bytes, at least fp8pa_workspace_bytes(); may be NULL
 *                when that is 0.  Contents on entry are ignored.
 *
 * Alignment: q, k_cache, v_cache and out 16 bytes; workspace 256 bytes;
 * block_table, seq_lens, scales, sinks and lse 4 bytes.
 * Device-side preconditions (not checked): 0 <= seq_lens[b] <= max_seq_len,
 * and block_table[b][j] in [0, num_blocks) for every page j that holds an
 * attended token.  A query whose position seq_lens[b] - q_len + i is
 * negative attends nothing and gets out 0 and lse -inf (the sink's logit
 * with sinks), so a batch may be padded with 0-token sequences.  Entries of pages holding no attended token are never
 * read and may be -1; cache bytes of tokens no row attends are never used
 * (they may hold NaN codes).
 * Returns FP8PA_ERR_WORKSPACE_TOO_SMALL when workspace_bytes is short and
 * FP8PA_ERR_HIP when a launch fails.
 */
fp8pa_status fp8pa_decode(const fp8pa_shape* shape, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_table,
                          const int32_t* seq_lens, const float* k_scale,
                          const float* v_scale, const float* sinks, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8pa_decode_noalloc: fp8pa_decode for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  It computes exactly what
 * fp8pa_decode computes, with the same plan and kernels, and takes the same
 * arguments minus the workspace: the split partials go to a static device
 * array of FP8PA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every
 * device it runs on until the process ends.  It allocates nothing, and the
 * array's device address is looked up once per device on the first call
 * there.  Every call on a device shares that device's array, so calls that
 * may overlap on one device (different streams, no ordering between them)
 * race and give undefined results; calls ordered on one stream are safe.
 * Returns FP8PA_ERR_WORKSPACE_TOO_SMALL when the plan's workspace
 * (fp8pa_workspace_bytes) exceeds FP8PA_NOALLOC_SCRATCH_BYTES, FP8PA_ERR_HIP
 * when the array's address cannot be obtained or a launch fails, and
 * otherwise what fp8pa_decode returns for the same arguments.
 */
#define FP8PA_NOALLOC_SCRATCH_BYTES (64u << 20)
fp8pa_status fp8pa_decode_noalloc(const fp8pa_shape* shape, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, const float* k_scale,
                                  const float* v_scale, const float* sinks, void* out, float* lse,
                                  void* stream);

/*
 * fp8pa_merge: the log-sum-exp merge of split-KV partials (FlashInfer PR
 * #5591, Summary: one LSE reducer after the split producers).  For each row
 * r < num_rows, with M = max(partial_lse[r, s], sink):
 *   out[r, :] = sum_s e^{lse_s - M} partial_o[r, s, :] / L,
 *   lse[r]    = M + ln L,   L = sum_s e^{lse_s - M} + e^{sink - M}.
 * A split with lse_s = -inf contributes nothing (its partial_o values are
 * ignored and may be NaN or garbage);
 * a row with no finite term gets out = 0, lse = -inf.
 *
 *   partial_o    float [num_rows, num_splits, head_dim]
 *   partial_lse  float [num_rows, num_splits], natural log
 *   sinks        float [num_q_heads] or NULL; row r uses sinks[r % num_q_heads]
 *   out          bf16  [num_rows, head_dim]
 *   lse          float [num_rows] or NULL
 * head_dim is 64, 128 or 256; num_splits >= 1; num_rows >= 0.  partial_o and
 * out 16-byte aligned, the rest 4-byte aligned.  This is the kernel
 * fp8pa_decode runs after its partial pass; it also merges partials that
 * another device computed over its own slice of each sequence.
 */
fp8pa_status fp8pa_merge(int32_t num_splits, int32_t num_rows, int32_t num_q_heads,
                         int32_t head_dim, const float* partial_o, const float* partial_lse,
                         const float* sinks, void* out, float* lse, void* stream);

/*
 * ---------------------------------------------------------------------------
 * The KV-cache writer: new tokens' bf16 keys and values into the E4M3 pages
 * fp8pa_decode reads.  The gist "Qwen3.8-27B ... 451K tokens of KV on a
 * single RTX 5090" (kernel reshape_and_cache_nvfp4_kernel) writes NVFP4
 * pages the same way: token t goes to slot slot_mapping[t], i.e. page
 * slot / block_tokens at position slot % block_tokens, a negative slot
 * meaning "skip", and each element is multiplied by the fp32 reciprocal of
 * its scale before encoding.  Here element x of kv head h is stored as
 * e4m3(x * (1 / scale_h)), the reciprocal and the product in fp32, rounded
 * to nearest with ties to even and saturated to +-448 (the FN format has no
 * infinity); a NaN element gives a NaN code.  fp8pa_decode then reads
 * decode(code) * scale_h.
 *
 * NVFP4 pools (kv_format = FP8PA_KV_NVFP4): each 16-element block of a
 * head's row becomes one E4M3 scale byte and 16 E2M1 codes, by the steps of
 * the quantizer the gist prints (nvfp4_utils.cuh, cvt_warp_fp16_to_fp4,
 * NVFP4 path) with the global scale g = fp32(1 / scale_h) the cache kernel
 * hands it: s = fp32(g * fp32(max|x| * fp32(1/6))), the scale byte = E4M3
 * of s (nearest, ties to even, saturating at 448), and the codes = E2M1 of
 * fp32(x * r) with r = fp32(1 / fp32(E4M3(byte) * fp32(1 / g))) (0 when the
 * byte decodes to 0), nearest with ties to even, saturated at 6, keeping
 * the sign bit.  The page forms these reciprocals with an approximate
 * instruction; this library uses correctly rounded division.  NaN inputs
 * are outside the format (their block's bytes are unspecified).
 *
 * MXFP8 pools (kv_format = FP8PA_KV_MXFP8): each 32-element block of a head's
 * row becomes one E8M0 scale byte and 32 E4M3 codes, by the OCP MX rule:
 * y = fp32(x * fp32(1 / scale_h)); the shared exponent X = floor(log2(max|y|))
 * - 8 (8 being E4M3's largest exponent), clamped to [-127, 127] (-127 for an
 * all-zero block); the scale byte X + 127; the codes e4m3(y * 2^-X), nearest
 * with ties to even and saturated to +-448.  NaN inputs are outside the
 * format.
 */
typedef struct fp8pa_write_shape {
  int64_t num_tokens;      /* T >= 0 rows of key, value and slot_mapping */
  int64_t key_stride;      /* elements between token rows of key: >= Hkv * D, a multiple of 8 */
  int64_t value_stride;    /* the same for value */
  int32_t num_kv_heads;    /* Hkv >= 1 */
  int32_t head_dim;        /* D: 64, 128 or 256 */
  int32_t block_tokens;    /* bt: tokens per page, a power of two in [1, 1024] */
  int32_t num_blocks;      /* pages in each pool, >= 1 */
  int32_t k_scale_count;   /* kg (per tensor) or Hkv * kg (per kv head), kg = max(k_groups, 1) */
  int32_t v_scale_count;   /* 1 or Hkv */
  int32_t k_groups;        /* as in fp8pa_shape: each key element is encoded against
                              the scale of its head_dim group */
  int32_t kv_layout;       /* FP8PA_LAYOUT_NHD or FP8PA_LAYOUT_HND, both pools */
  int32_t kv_format;       /* FP8PA_KV_E4M3, FP8PA_KV_NVFP4 or FP8PA_KV_MXFP8 (the last two
                              with k_groups <= 1) */
  int64_t kv_page_stride;  /* as in fp8pa_shape */
} fp8pa_write_shape;

/*
 * fp8pa_cache_write: writes every token t < T whose slot lies in
 * [0, num_blocks * bt) into both pools; other slots are skipped.
 *
 *   key, value    bf16 [T, Hkv, D], token rows key_stride / value_stride
 *                 elements apart (16-byte aligned)
 *   slot_mapping  int64 [T]
 *   k_scale       float [k_scale_count]; v_scale float [v_scale_count]
 *   k_cache       e4m3 [num_blocks, bt, Hkv, D] (8-byte aligned), or
 *                 [num_blocks, Hkv, bt, D] with kv_layout = FP8PA_LAYOUT_HND, or NVFP4
 *                 pages (see FP8PA_KV_NVFP4) or MXFP8 pages; pages kv_page_stride bytes apart when it
 *                 is not 0; v_cache alike
 *
 * Only the slots named are written.  Two tokens with the same slot race
 * (either may win).  All pointers are device pointers owned by the caller;
 * work is queued on `stream`.  Returns FP8PA_ERR_INVALID_ARG /
 * FP8PA_ERR_UNSUPPORTED / FP8PA_ERR_MISALIGNED for bad host-known
 * arguments (nothing is queued then), FP8PA_ERR_HIP if the launch fails.
 */
fp8pa_status fp8pa_cache_write(const fp8pa_write_shape* shape, const void* key, const void* value,
                               const int64_t* slot_mapping, const float* k_scale,
                               const float* v_scale, void* k_cache, void* v_cache, void* stream);

/* Static text for a status code. */
const char* fp8pa_status_string(fp8pa_status status);

/* Library version and build description (static text). */
const char* fp8pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8PA_H_ */
