/*
 * mqa.h - C ABI of libmqa: fp8 paged MQA logits and per-row top-k on MI355X (gfx950),
 * with the non-paged (prefill) form of the logits, the indexer K-cache write and the
 * sparse MLA decode over the selected positions.
 *
 * The operation is the decode step of the sparse-attention indexer described on
 * the stepcodex.com issue page "[Bug] aiter ops triton attention pa_mqa_logits"
 * (section "Minimal reproduction": the torch reference function, which reads
 * block_size from the cache shape and walks the blocks of a request, and the
 * reproducer's top-k comparison; section "Observations while narrowing it down"
 * for the block sizes in use and the index head counts).
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer (hipMalloc or torch CUDA tensor memory),
 *     except `shape`, which is a host pointer read during the call only.
 *   - The caller owns all memory. The library never allocates, frees, synchronises,
 *     or reads device memory from the host. All work is enqueued on `stream`
 *     (0 = the default stream), so calls are asynchronous and capturable into a
 *     HIP graph.
 *   - Arguments are validated on the host before anything is enqueued. A rejected
 *     call returns a nonzero status and enqueues nothing. MQA_ERR_HIP reports a
 *     launch failure seen by hipGetLastError after the launch.
 *   - Values that live on the device (context lengths, block-table entries) cannot
 *     be checked on the host. The kernels clamp them so that no access leaves the
 *     buffers described by `shape`:
 *       ctx is read as min(max(ctx, 0), block_table_stride * block_size,
 *       max_model_len); a block-table entry outside [0, num_blocks) yields NaN
 *       logits for the tokens of that block instead of a memory access.
 *   - Calls are reentrant: no mutable global state, except the static scratch of
 *     mqa_topk_noalloc (see there).
 */
#ifndef MQA_H
#define MQA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  MQA_OK = 0,
  MQA_ERR_NULL = 1,        /* a required pointer is NULL */
  MQA_ERR_SHAPE = 2,       /* a size is negative, zero where it may not be, or overflows */
  MQA_ERR_UNSUPPORTED = 3, /* a valid shape outside the supported domain (below) */
  MQA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than mqa_topk_workspace_bytes */
  MQA_ERR_HIP = 5,         /* the HIP runtime reported an error at launch */
  MQA_ERR_SCRATCH = 6      /* mqa_topk_noalloc: the problem needs more than the static scratch */
};

/*
 * Problem shape (host struct).
 *   batch               B, number of requests (>= 0; 0 enqueues nothing; at most 8192
 *                       for mqa_paged_logits)
 *   next_n              N, decode rows per request (speculative depth + 1), 1..4
 *   heads               H, index query heads, a multiple of 16 in [16, 128]
 *   head_dim            D, must be 128
 *   block_size          S, tokens per KV block: a power of two in [1, 65536]
 *   block_table_stride  W, int32 elements (blocks) per block-table row (>= 1);
 *                       W * S <= 2^31 - 1
 *   num_blocks          blocks in the KV cache (>= 1); for S > 1, num_blocks * S
 *                       <= 2^31 - 1
 * Row r of the logits and of the indices is decode row j of request b, r = b*N + j.
 */
typedef struct mqa_shape {
  int32_t batch;
  int32_t next_n;
  int32_t heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t block_table_stride;
  int64_t num_blocks;
} mqa_shape;

/*
 * mqa_paged_logits - indexer logits for every decode row and every position.
 *
 * Definition (stepcodex.com pa_mqa_logits issue, "Minimal reproduction", the torch
 * reference): for row r = b*N + j with context length ctx = context_lens[b], position t
 * is visible iff t <= ctx - N + j (the row's own position; it implies t < ctx). Token t
 * is slot t % S of block block_tables[b*W + t / S]; for a visible t that is cache row
 * p = block_tables[b*W + t / S] * S + t % S, and:
 *     k      = e4m3fn bytes kv_cache[p*132 + 0 .. 127]          (OCP E4M3, bias 7)
 *     scale  = little-endian fp32 at kv_cache[p*132 + 128 .. 131]
 *     out[r*max_model_len + t] = sum_h weights[r*H + h] * relu(scale * (q[b,j,h,:] . k))
 * Every other slot of the row, t in [visible, max_model_len), is written with -inf.
 *
 *   q               uint8  [B, N, H, 128]   e4m3fn, contiguous, 16-byte aligned
 *   kv_cache        uint8  [num_blocks, S, 132] per token: 128 e4m3fn key bytes, then
 *                                            the fp32 scale; rows are 4-byte aligned
 *                                            (the pointer must be too)
 *   weights         float  [B*N, H]         16-byte aligned
 *   context_lens    int32  [B]              4-byte aligned
 *   block_tables    int32  [B, W]           4-byte aligned
 *   max_model_len   L >= 1, the length of each output row; B * N * (ceil(L/64) + 1)
 *                   must stay below 2^31 (the work is counted in 32-bit units), else
 *                   MQA_ERR_UNSUPPORTED
 *   out             float  [B*N, L]         every element is written; 4-byte aligned (rows
 *                                            that are 16-byte aligned are written faster)
 *   shape, stream   see above
 * A pointer with less than the alignment stated is rejected with MQA_ERR_UNSUPPORTED.
 * Accuracy: fp8 x fp8 products are exact, accumulated in fp32; relu, weight and head
 * sum in fp32. Results agree with the exact definition to 5e-3 + 1e-3*|logit| on the
 * supported distributions; NaN key codes or NaN/Inf scales propagate as NaN.
 * Returns MQA_OK, MQA_ERR_NULL, MQA_ERR_SHAPE, MQA_ERR_UNSUPPORTED or MQA_ERR_HIP.
 */
int mqa_paged_logits(const uint8_t* q, const uint8_t* kv_cache, const float* weights,
                     const int32_t* context_lens, const int32_t* block_tables,
                     int32_t max_model_len, float* out, const mqa_shape* shape,
                     hipStream_t stream);

/*
 * mqa_topk - positions of the k largest logits of each row's visible prefix.
 *
 * Definition (stepcodex.com pa_mqa_logits issue, "Minimal reproduction": the reproducer
 * keeps k = min(2048, ctx) positions per row with topk and compares them as sets): row r
 * has visible = max(0, min(ctx - N + j + 1, L)) positions. The call writes
 * idx[r*k + 0 .. m-1], m = min(k, visible), with the m positions t < visible whose
 * logits are largest, in unspecified order (a set), and idx[r*k + m .. k-1] = -1.
 * Order: larger logit first; equal logits (-0.0 equals +0.0) by lower position first.
 * NaN logits are ordered by their bit patterns (positive NaN above +inf).
 *
 *   logits          float  [B*N, L]   as written by mqa_paged_logits (only the visible
 *                                     prefix of each row is read), 4-byte aligned
 *   context_lens    int32  [B]        4-byte aligned
 *   max_model_len   L, the row stride of logits. Not among the two arguments the
 *                   operation itself needs (logits and context lengths): it is the
 *                   row stride, and it bounds the visible prefix like the logits call
 *   k               1 .. 2048
 *   idx             int32  [B*N, k]   4-byte aligned
 *   workspace       device scratch of at least mqa_topk_workspace_bytes(shape,
 *                   max_model_len, k) bytes, 16-byte aligned (may be NULL when that
 *                   size is 0, i.e. max_model_len <= 32768). It must hold zeros before
 *                   its first use (fill it once, e.g. hipMemset or torch.zeros, outside
 *                   any captured graph); every call returns it to zero before it ends,
 *                   in stream order, so the same workspace serves any number of calls of
 *                   any shape that fits it, captured into graphs or not. Calls that
 *                   overlap in time must not share a workspace.
 * Returns MQA_OK, MQA_ERR_NULL, MQA_ERR_SHAPE, MQA_ERR_UNSUPPORTED,
 * MQA_ERR_WORKSPACE or MQA_ERR_HIP.
 */
int mqa_topk(const float* logits, const int32_t* context_lens, int32_t max_model_len,
             int32_t k, int32_t* idx, const mqa_shape* shape, void* workspace,
             size_t workspace_bytes, hipStream_t stream);

/*
 * mqa_topk_noalloc - mqa_topk without a workspace argument and without any allocation.
 *
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. The result is that of mqa_topk with the
 * same arguments (the same kernels run); the scratch that mqa_topk takes from its
 * workspace argument is a static device array of the library instead, 64 MiB on each
 * device the library runs on, zero when the library is loaded and held until the process
 * ends. A problem whose mqa_topk_workspace_bytes exceeds 64 MiB is rejected with
 * MQA_ERR_SCRATCH before anything is enqueued (with max_model_len > 32768 every row needs
 * about 80 KB, so up to ~800 rows per call; with max_model_len <= 32768 none is needed).
 * The call allocates nothing: the array's device address is looked up once per device
 * (hipGetSymbolAddress) on the first call that needs it. Every call on a device shares
 * that device's array and, like mqa_topk with its workspace, returns it to zero before it
 * ends: calls that overlap in time on one device - on different streams, or from
 * different threads - race and give undefined results. Calls in one stream are ordered
 * and safe.
 * Arguments, layouts and other errors as mqa_topk; MQA_ERR_HIP also reports a failed
 * symbol lookup.
 */
int mqa_topk_noalloc(const float* logits, const int32_t* context_lens, int32_t max_model_len,
                     int32_t k, int32_t* idx, const mqa_shape* shape, hipStream_t stream);

/*
 * mqa_logits - the same logits over contiguous keys for M query rows with per-row key
 * windows (the non-paged, prefill form).
 *
 * Definition: the quantity of mqa_paged_logits; the stepcodex.com pa_mqa_logits issue
 * ("Observations while narrowing it down") names the prefill kernel that computes it for
 * many query rows at once (fp8_mqa_logits) but not its signature. Here:
 *     out[i*out_stride + j] = sum_h weights[i*H + h] * relu(k_scale[j] * (q[i,h,:] . k[j,:]))
 *                             if ks[i] <= j < ke[i], and -inf for every other j < n,
 * with ks[i], ke[i] read as clamped to [0, n] (an empty window leaves the row -inf).
 *
 *   q           uint8 [m, H, 128]  e4m3fn, 16-byte aligned
 *   k           uint8 [n, 128]     e4m3fn, 16-byte aligned
 *   k_scale     float [n]          per-key dequant scale
 *   weights     float [m, H]       16-byte aligned
 *   ks, ke      int32 [m]
 *   out         float [m, out_stride], out_stride >= n; elements [n, out_stride) of a row
 *               are not touched
 *   m >= 0 (0 enqueues nothing), 1 <= n <= 2^29, heads a multiple of 16 in [16, 64]
 * Accuracy as mqa_paged_logits (exact fp8 products, fp32 accumulation).
 * Returns MQA_OK, MQA_ERR_NULL, MQA_ERR_SHAPE, MQA_ERR_UNSUPPORTED or MQA_ERR_HIP.
 */
int mqa_logits(const uint8_t* q, const uint8_t* k, const float* k_scale, const float* weights,
               const int32_t* ks, const int32_t* ke, float* out, int64_t out_stride, int32_t m, int32_t n,
               int32_t heads, hipStream_t stream);

/* Element types of the keys given to mqa_indexer_k_write. */
enum { MQA_DTYPE_BF16 = 0, MQA_DTYPE_F32 = 1 };

/*
 * mqa_indexer_k_write - quantise keys into the cache rows mqa_paged_logits reads.
 *
 * Row format (stepcodex.com pa_mqa_logits issue, "Minimal reproduction": the reference
 * reads bytes [0, 128) of a token's row as e4m3fn codes and bytes [128, 132) as one
 * little-endian fp32 scale, and dequantises code * scale). The page does not state how
 * a writer picks the scale; this call maps the row's largest magnitude onto the largest
 * finite code:
 *     amax  = max_i |k[t, i]|
 *     scale = amax / 448 in fp32, correctly rounded (scale = 1 when amax = 0)
 *     code  = e4m3fn(k[t, i] / scale): the fp32 quotient, correctly rounded, then the
 *             nearest e4m3fn value, ties to even (so |code| <= 448; a NaN key makes
 *             the row NaN, with the scale written as the quiet NaN 0x7FC00000; an
 *             infinite key gives an infinite scale; -0.0 keeps its sign, code 0x80)
 * and writes row slot_mapping[t] (row blk * block_size + offset of a blocked cache):
 *     kv_cache[slot*132 + 0 .. 127] = codes, kv_cache[slot*132 + 128 .. 131] = scale.
 * Tokens whose slot lies outside [0, num_slots) are skipped (negative slots mark
 * padding). Two tokens mapped to one slot race; the result is one of them.
 *
 *   k             [num_tokens, 128] contiguous, bf16 (MQA_DTYPE_BF16) or fp32
 *                 (MQA_DTYPE_F32), 16-byte aligned
 *   k_dtype       MQA_DTYPE_BF16 or MQA_DTYPE_F32
 *   num_tokens    T >= 0 (0 enqueues nothing)
 *   slot_mapping  int64 [T], 8-byte aligned
 *   kv_cache      uint8 [num_slots, 132], 4-byte aligned
 *   num_slots     rows of the cache (num_blocks * block_size), >= 1
 * Returns MQA_OK, MQA_ERR_NULL, MQA_ERR_SHAPE, MQA_ERR_UNSUPPORTED or MQA_ERR_HIP.
 */
int mqa_indexer_k_write(const void* k, int32_t k_dtype, int64_t num_tokens, const int64_t* slot_mapping,
                        uint8_t* kv_cache, int64_t num_slots, hipStream_t stream);

/*
 * Shape of a sparse MLA decode call. rows = batch * next_n query rows; row r = b*N + j
 * belongs to request b.
 */
typedef struct mqa_mla_shape {
  int32_t batch;              /* B requests */
  int32_t next_n;             /* N query tokens per request (1..4 in the pages' use; any >= 1) */
  int32_t heads;              /* query heads per row: 16 */
  int32_t head_dim;           /* latent row width in bytes / codes: 576 */
  int32_t v_dim;              /* value width: 512 (the first 512 dims of a latent row) */
  int32_t block_size;         /* S tokens per cache block, a power of two up to 65536 */
  int32_t block_table_stride; /* W entries per block-table row */
  int32_t topk;               /* entries per row of indices */
  int64_t num_blocks;         /* blocks in kv_cache */
} mqa_mla_shape;

/*
 * mqa_sparse_mla_decode - attention of each decode row over the positions the indexer
 * selected for it (sparse MLA decode).
 *
 * Sources: the stepcodex.com pa_mqa_logits issue, "Downstream impact" (the positions the
 * top-k keeps are the ones the sparse attention attends); the chat-gpts.plus summary
 * (post 69330) of the aiter MLA decode issue, "问题场景" and "环境排查" (fp8 q and KV cache,
 * 16 query heads per latent KV head, 1 to 4 query tokens per request); vLLM pull request
 * 31282, "The Bug" (one token per cache page). The pages leave the row width, the scale
 * placement and the list form open; this call reads them as:
 *   q            [rows, 16, 576] e4m3fn codes, dequantised as code * q_scale
 *   kv_cache     [num_blocks, S, 576] e4m3fn codes (576 = 512 compressed + 64 rotary dims,
 *                DeepSeek-V3's sizes), dequantised as code * kv_scale
 *   indices      [rows, topk] int32 positions of request b (the layout mqa_topk writes);
 *                a negative entry is padding; a position listed twice is attended twice
 *   block_tables [B, W] int32: position t is slot t % S of block block_tables[b*W + t/S]
 * and computes, over the row's listed positions t,
 *   score(h, t) = sm_scale * q_scale * kv_scale * (q[r,h,:] . k_t)
 *   out[(r*16 + h)*512 + c] = kv_scale * sum_t softmax_t(score(h, .)) * k_t[c], c < 512
 *   lse[r*16 + h] = log(sum_t exp(score(h, t)))   (natural log; lse may be NULL)
 * A row with no listed position gets out = 0 and lse = -inf. A listed position at or past
 * W*S, or whose block-table entry lies outside [0, num_blocks), makes its row NaN (out and
 * lse); no access leaves the described buffers.
 *
 * Precision: the 576-term dot products are exact (fp8 codes as f16, fp32 accumulation of
 * exact products, rounded as the hardware sums them); softmax in fp32 with probabilities
 * rounded to f16 (relative 2^-11) for the value contraction.
 *
 * Ownership: every pointer is a device pointer owned by the caller; shape is a host
 * struct. workspace (16-byte aligned, at least mqa_sparse_mla_workspace_bytes(shape)
 * bytes; may be NULL when that is 0) holds per-split partial results and is fully
 * rewritten by each call. Nothing is allocated or synchronised; the work is enqueued on
 * stream (capturable into a graph).
 *
 * Errors: MQA_ERR_NULL (shape, q, kv_cache, indices, block_tables or out NULL with rows >
 * 0), MQA_ERR_SHAPE (negative batch, next_n, topk, block_size, stride or num_blocks < 1),
 * MQA_ERR_UNSUPPORTED (heads != 16, head_dim != 576, v_dim != 512, block_size not a power
 * of two up to 65536, W*S or num_blocks*S at or above 2^31, rows > 65535, topk > 2^20,
 * q / kv_cache / out / workspace not 16-byte aligned, indices / block_tables / lse not
 * 4-byte aligned), MQA_ERR_WORKSPACE, MQA_ERR_HIP.
 */
int mqa_sparse_mla_decode(const uint8_t* q, float q_scale, const uint8_t* kv_cache, float kv_scale,
                          const int32_t* indices, const int32_t* block_tables, float sm_scale, float* out,
                          float* lse, const mqa_mla_shape* shape, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Workspace size for mqa_sparse_mla_decode with this shape on the current device (0 when
 * none is needed or the shape is invalid). */
size_t mqa_sparse_mla_workspace_bytes(const mqa_mla_shape* shape);

/* Workspace size for mqa_topk with this shape, L and k (0 when the shape is invalid). */
size_t mqa_topk_workspace_bytes(const mqa_shape* shape, int32_t max_model_len, int32_t k);

/* Static description of a status code (never NULL). */
const char* mqa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MQA_H */
