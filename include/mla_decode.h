/*
 * Paged absorbed-MLA decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libmla_decode.so.  Every entry point takes plain device pointers
 * and sizes, enqueues its work on the given HIP stream and returns a status
 * code; nothing synchronises with the host, and nothing is allocated: the
 * caller owns every buffer, including the decode workspace.  All argument
 * checks happen on the host before any launch, so a non-zero status means
 * nothing was enqueued.  Calls on different streams may overlap; a workspace
 * must not be shared by two calls in flight at the same time.
 *
 * Sources: three vLLM pull-request digest pages (prhub.com.cn):
 *   PR #52188 "support Kimi-K3 DSpark speculative decoding with DCP",
 *   PR #54012 "MLA decode with DCP switches to FlashInfer's native CP mask",
 *   PR #48180 "TokenSpeed MLA backend gains DCP and Eagle support".
 * Section names below are those pages' sections (summary, motivation,
 * implementation breakdown, key files, key source snippets, review
 * highlights, risks and impact).
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Widths of absorbed MLA: 512 latent + 64 rope per query head and per KV row
 * (PR #54012 page, key source snippets: kv_lora_rank 512, rope dim 64,
 * query [.., heads, 576], output [.., heads, 512]). */
#define MLA_D_QK 576
#define MLA_D_V 512

/* Slot value for positions a rank must not write (PR #52188 page, key source
 * snippets, cp_local_slot).  The pages do not print its value; -1 cannot
 * collide with a real slot. */
#define MLA_PAD_SLOT_ID (-1LL)

/* LSE bases.  Base e is the contract of the CuTeDSL DCP path (PR #54012
 * page, implementation breakdown: lse_base_on_e becomes true); base 2 is
 * TokenSpeed's (PR #48180 page, implementation breakdown). */
#define MLA_LSE_BASE_E 0
#define MLA_LSE_BASE_2 1

/* Status codes. */
#define MLA_OK 0
#define MLA_ERR_INVALID_ARG 1  /* a null pointer, a size or index out of range, a workspace too small */
#define MLA_ERR_UNSUPPORTED 2  /* reserved: a valid request this library does not implement (no call returns it today) */
#define MLA_ERR_HIP 3          /* the HIP runtime refused one of this call's launches (that launch's own status) */

/* Short static description of a status code; never NULL. */
const char* mla_status_string(int status);

/*
 * Bytes of device workspace mla_decode needs for these sizes on the current
 * device (0 when none): enough for every decode entry point (bf16 or FP8
 * cache, and mla_decode_varlen with q_len the largest query length, whose
 * work split can differ).  max_seq_len only sizes the work split; any upper
 * bound works.  Returns 0 for invalid sizes.
 */
size_t mla_decode_workspace_size(int B, int q_len, int H, int max_seq_len);

/*
 * One rank's absorbed MLA decode over its paged latent KV cache.
 *
 * What is computed (PR #54012 page, implementation breakdown and key source
 * snippets: the native-DCP kernel receives rank-local seq_lens together with
 * the global causal lengths, cp_world and cp_rank and masks every query row
 * itself; PR #52188 page, key source snippets: the per-row prefix and its
 * round-robin rank-local length; PR #48180 page, key source snippets: the
 * same contract for TokenSpeed with causal_seqs):
 *   For request b, query row j < q_len, head h, the scores are
 *     s_t = scale * sum_{d<576} q[b,j,h,d] * kv[row(b,t), d]
 *   over the rank-local keys t < n(b,j), where
 *     causal:     G = max(tot_b - (q_len-1-j), 0),
 *                 n(b,j) = min(seq_lens[b], ceil(max(G - cp_rank, 0) / cp_world)),
 *                 tot_b = causal_seqlens_global[b] (or seq_lens[b] when that
 *                 pointer is NULL, allowed only for cp_world == 1);
 *     non-causal: n(b,j) = seq_lens[b] for every row (a draft block).
 *   out[b*q_len+j, h, :] = softmax(s) @ kv[row(b,t), 0:512]   (bf16, RNE)
 *   lse[b*q_len+j, h]    = log of sum_t exp(s_t), natural log for
 *                          MLA_LSE_BASE_E, log2 for MLA_LSE_BASE_2.
 *   A row with n(b,j) == 0 gets out = 0 and lse = -inf.
 *   Local key t lives at physical row
 *     block_table[b*max_blocks + t/block_size]*block_size + t%block_size.
 *   The rank's keys are the global positions t*cp_world + cp_rank
 *   (round-robin, interleave 1: the native CP mask requires it, PR #54012
 *   page, implementation breakdown).
 *
 * Layouts (all contiguous, row-major, device memory):
 *   q                     [B, q_len, H, 576] bf16
 *   kv_cache              [num_blocks, block_size, 576] bf16 (512 latent, then 64 rope)
 *   block_table           [B, max_blocks] int32
 *   seq_lens              [B] int32, rank-local lengths
 *   causal_seqlens_global [B] int32 or NULL, global lengths including the
 *                         request's own q_len query tokens
 *   out                   [B*q_len, H, 512] bf16
 *   lse                   [B*q_len, H] float32, or NULL to skip it
 *   workspace             >= mla_decode_workspace_size(B, q_len, H, max_seq_len) bytes
 * Arguments: causal is 0 or 1; lse_base is MLA_LSE_BASE_E or MLA_LSE_BASE_2;
 * 0 <= cp_rank < cp_world.  B == 0 is a no-op.
 * Device-side preconditions (not checked on the host, which cannot read
 * device memory without a sync): seq_lens[b] <= max_blocks*block_size.
 * Out-of-range block ids are guarded in the kernel: such keys read as zero
 * rows instead of faulting, and the result for that request is undefined.
 * Errors: MLA_ERR_INVALID_ARG for null pointers, sizes < 1 (B < 0),
 * cp_rank outside [0, cp_world), causal with cp_world > 1 and a NULL global
 * pointer, an unknown lse_base, a non-finite scale, or a workspace smaller
 * than required; MLA_ERR_HIP if a launch fails.
 */
int mla_decode(const void* q, const void* kv_cache, const int32_t* block_table,
               const int32_t* seq_lens, const int32_t* causal_seqlens_global,
               int B, int q_len, int H, int num_blocks, int block_size, int max_blocks,
               int max_seq_len, int cp_world, int cp_rank, int causal, float scale,
               int lse_base, void* out, float* lse, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/*
 * mla_decode for ranks that hold their keys in segments of cp_interleave
 * positions: segment k of a request's global positions (positions
 * k*cp_interleave .. k*cp_interleave + cp_interleave - 1) belongs to rank
 * k % cp_world, and the rank's local key t is the t-th position it owns
 * (PR #52188 page, key source snippets, cp_local_slot, and the rank-local
 * length it prints for an interleave).  The causal bound of row j becomes
 *   G = max(tot_b - (q_len-1-j), 0),
 *   n(b,j) = min(seq_lens[b], (G / (I*W))*I + min(max(G % (I*W) - r*I, 0), I))
 * with I = cp_interleave, W = cp_world, r = cp_rank; everything else is as in
 * mla_decode, which is this call with cp_interleave = 1.  (The native CP
 * mask of the PR #54012 page supports interleave 1 only; this is the
 * generalisation the slot mapping already describes.)
 * Errors: those of mla_decode, and MLA_ERR_INVALID_ARG for cp_interleave < 1
 * or cp_interleave*cp_world > 2^30.
 */
int mla_decode_interleaved(const void* q, const void* kv_cache, const int32_t* block_table,
                           const int32_t* seq_lens, const int32_t* causal_seqlens_global,
                           int B, int q_len, int H, int num_blocks, int block_size, int max_blocks,
                           int max_seq_len, int cp_world, int cp_rank, int cp_interleave, int causal,
                           float scale, int lse_base, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * mla_decode for a batch whose requests have different query lengths
 * (varlen).  The query tokens of all requests are packed: request b owns
 * tokens query_start_loc[b] .. query_start_loc[b+1]-1 of q, so its query
 * length is q_len_b = query_start_loc[b+1] - query_start_loc[b] (0 allowed).
 * Row j < q_len_b of request b applies the causal prefix with its own length
 * (PR #52188 page, key source snippets: tot - (query_len - 1 - j); summary:
 * the backends declare support for batches of different query lengths,
 * supports_dcp_with_varlen):
 *   G = max(tot_b - (q_len_b-1-j), 0) and the bound of mla_decode_interleaved;
 * non-causal rows see seq_lens[b].  Outputs follow the tokens:
 *   out[(query_start_loc[b]+j)*H + h, :], lse[(query_start_loc[b]+j)*H + h].
 * Layouts: q [T, H, 576] bf16 and out [T, H, 512] bf16, lse [T, H] float32
 * (T = query_start_loc[B]); query_start_loc [B+1] int32 in device memory,
 * non-decreasing, starting at 0.  max_q_len (host) must be at least every
 * q_len_b; it sizes the work split and the workspace:
 *   mla_decode_workspace_size(B, max_q_len, H, max_seq_len).
 * Device-side precondition (not checked): q_len_b <= max_q_len; rows of a
 * longer request past max_q_len*H are left unwritten.
 * Errors: those of mla_decode_interleaved (with q_len = max_q_len), and
 * MLA_ERR_INVALID_ARG for a NULL query_start_loc when B > 0.
 */
int mla_decode_varlen(const void* q, const int32_t* query_start_loc, int max_q_len, const void* kv_cache,
                      const int32_t* block_table, const int32_t* seq_lens, const int32_t* causal_seqlens_global,
                      int B, int H, int num_blocks, int block_size, int max_blocks, int max_seq_len,
                      int cp_world, int cp_rank, int cp_interleave, int causal, float scale, int lse_base,
                      void* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mla_kv_write into an FP8 latent cache (the write side of mla_decode_fp8;
 * PR #54012 page, key source snippets: the cache dtype and its scales).
 * Each bf16 value v of a new row is stored as the E4M3 code of the
 * correctly rounded float32 quotient v / kv_scale: the nearest E4M3 value,
 * ties to the even code, magnitudes from 448 up and infinities saturated to
 * +-448 (0x7E/0xFE), NaN as 0x7F, the sign of zero kept.
 * kv_new: [n_rows, 576] bf16 (16-byte aligned); slots: [n_rows] int64 as
 * for mla_kv_write (pad, negative and past-the-end slots write nothing);
 * kv_cache: [num_blocks, block_size, 576] bytes (16-byte aligned).  Rows with
 * the same slot: unspecified which one stays.
 * Errors: those of mla_kv_write, and MLA_ERR_INVALID_ARG for a kv_scale that
 * is not finite and positive.
 */
int mla_kv_write_fp8(const void* kv_new, const int64_t* slots, int64_t n_rows, float kv_scale, void* kv_cache,
                     int num_blocks, int block_size, hipStream_t stream);

/*
 * mla_decode_interleaved over an FP8 latent cache (PR #54012 page, key
 * source snippets: the backend's cache dtype and its bmm1/bmm2 scales, and
 * the output scale handed to the decode kernel).  kv_cache holds
 * [num_blocks, block_size, 576] bytes, each an E4M3 code (OCP 8-bit float:
 * 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, 0x7f
 * and 0xff are NaN, largest value 448); the key/value row is each code's
 * value times kv_scale, one factor for the whole cache.  Scores are
 * scale * q . (kv_scale * code), the output is the softmax-weighted sum of
 * the dequantised value rows, and the LSE is that of the scaled scores.  The
 * query, output, LSE, workspace and every other argument are those of
 * mla_decode_interleaved (its workspace size query applies unchanged).
 * Errors: those of mla_decode_interleaved, and MLA_ERR_INVALID_ARG for a
 * kv_scale that is not finite and positive.
 */
int mla_decode_fp8(const void* q, const void* kv_cache, float kv_scale, const int32_t* block_table,
                   const int32_t* seq_lens, const int32_t* causal_seqlens_global, int B, int q_len, int H,
                   int num_blocks, int block_size, int max_blocks, int max_seq_len, int cp_world, int cp_rank,
                   int cp_interleave, int causal, float scale, int lse_base, void* out, float* lse,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Size of the device array mla_decode_noalloc uses as its workspace: 96 MiB
 * on each GPU the library runs on, held until the process ends.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)96 * 1024 * 1024)

/*
 * mla_decode for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, serving loops that forbid
 * allocation, harnesses without an allocator.  Same arguments, layouts,
 * results and errors as mla_decode, without workspace and workspace_bytes:
 * the split-KV partials live in a fixed device array of
 * MLA_NOALLOC_SCRATCH_BYTES per GPU instead.  The call allocates nothing and
 * calls no allocating routine; its first call on a device looks up that
 * device's array once.  The caller still owns and passes every input and
 * output.
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that overlap
 * on one GPU, on any streams, race and must be serialised by the caller.
 * Errors: those of mla_decode, and MLA_ERR_INVALID_ARG when the sizes need
 * more than MLA_NOALLOC_SCRATCH_BYTES (at most mla_decode_workspace_size(B,
 * q_len, H, max_seq_len) bytes; e.g. B = 16, q_len = 16, H = 128 and a
 * 131072-key bound need 69 MB); MLA_ERR_HIP if the array's address cannot be
 * obtained.
 */
int mla_decode_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                       const int32_t* seq_lens, const int32_t* causal_seqlens_global,
                       int B, int q_len, int H, int num_blocks, int block_size, int max_blocks,
                       int max_seq_len, int cp_world, int cp_rank, int causal, float scale,
                       int lse_base, void* out, float* lse, hipStream_t stream);

/*
 * Profiling aid (not part of the computation): for the calling host thread,
 * record `start` at the start and `stop` at the end of the split-KV
 * attention kernel of each following mla_decode call (the kernel is then
 * launched with hipExtLaunchKernel, which records both events as part of its
 * dispatch on that call's stream).  Pass two
 * NULLs to stop.  The events are created and owned by the caller; each call
 * re-records them, so a caller timing several calls sets a fresh pair before
 * each.  Returns MLA_ERR_INVALID_ARG if exactly one of them is NULL.
 */
int mla_profile_attention_events(hipEvent_t start, hipEvent_t stop);

/*
 * A measurement helper, not part of the decode path: runs a bare bf16 MFMA
 * loop (v_mfma_f32_32x32x16_bf16, four independent accumulation chains per
 * wave, iters steps of four MFMAs) on `workgroups` workgroups of 256 threads,
 * the achievable matrix rate beside the published peak.  Work per launch:
 * workgroups * 4 waves * iters * 4 * 32768 flop.  out (device, float32,
 * workgroups * 256 values, caller-owned) receives 64 * iters in every
 * element.  Returns MLA_ERR_INVALID_ARG for workgroups or iters outside
 * [1, 2^20] or a NULL out.
 */
int mla_probe_mfma(int workgroups, int iters, float* out, hipStream_t stream);

/*
 * Merge partial attention results of disjoint key sets (the ranks' shards)
 * by their LSE (PR #54012 page, implementation breakdown: the CP path returns
 * a natural-log LSE and the bases must agree before the cross-rank merge;
 * PR #48180 page, implementation breakdown: the DCP decode output is merged
 * after the kernel).  With M = max_i lse_i and beta the base:
 *   w_i = beta^(lse_i - M),  out = sum_i w_i out_i / sum_i w_i,
 *   lse = M + log_beta(sum_i w_i);
 * partials with lse = -inf get weight 0; if all are -inf the result is
 * out = 0, lse = -inf.
 * partials: host array of n_parts device pointers, each [rows, H, 512] bf16.
 * lses:     host array of n_parts device pointers, each [rows, H] float32.
 * out: [rows, H, 512] bf16; lse: [rows, H] float32 or NULL.
 * 1 <= n_parts <= 64.  The host arrays are read during the call only.
 * Errors: MLA_ERR_INVALID_ARG for null pointers, n_parts outside [1, 64],
 * rows < 0, H < 1, or an unknown lse_base; MLA_ERR_HIP if the launch fails.
 */
int mla_merge_lse(const void* const* partials, const float* const* lses, int n_parts,
                  int rows, int H, int lse_base, void* out, float* lse, hipStream_t stream);

/*
 * Rank-local KV slot of each position, or MLA_PAD_SLOT_ID (PR #52188 page,
 * key source snippets, cp_local_slot; implementation breakdown: the DFlash
 * input preparation takes the virtual block index pos // (block_size*cp_world)
 * and applies the slot mapping to context and query positions).  For
 * position pos = positions[b*n + i]:
 *   span = block_size*cp_world, v = pos / span, off = pos % span;
 *   pad if i >= num_valid[b] (the rejected suffix), pos < 0, or v >= max_blocks;
 *   blk = block_table[b*max_blocks + v];
 *   cp_world == 1: slot = blk*block_size + off;
 *   else pad unless (off / cp_interleave) % cp_world == cp_rank, and then
 *     slot = blk*block_size + (off / (cp_interleave*cp_world))*cp_interleave
 *            + off % cp_interleave.
 * positions: [B, n] int64; num_valid: [B] int32 or NULL (all valid);
 * block_table: [B, max_blocks] int32; slots: [B, n] int64.  Bit-exact integer
 * arithmetic in 64 bits.
 * Errors: MLA_ERR_INVALID_ARG for null pointers (when B*n > 0), B or n < 0,
 * max_blocks < 1, block_size < 1, cp_world < 1, cp_rank outside
 * [0, cp_world), cp_interleave < 1 or block_size not a multiple of
 * cp_interleave; MLA_ERR_HIP if the launch fails.
 */
int cp_local_slot(const int64_t* positions, const int32_t* num_valid, int B, int n,
                  const int32_t* block_table, int max_blocks, int block_size,
                  int cp_world, int cp_rank, int cp_interleave, int64_t* slots,
                  hipStream_t stream);

/*
 * Store new latent KV rows in a rank's paged cache at their rank-local slots
 * (PR #52188 page, key source snippets, cp_local_slot: a rank writes the
 * draft's KV only at the slots it owns and gets the pad slot for the others,
 * so that it never overwrites another rank's rows; implementation
 * breakdown: the DFlash input preparation applies the slot mapping to the
 * draft's context and query KV).  For every i < n_rows:
 *   if 0 <= slots[i] < num_blocks*block_size:
 *     kv_cache[slots[i] / block_size][slots[i] % block_size][:] = kv_new[i][:]
 *   otherwise (MLA_PAD_SLOT_ID, any negative slot, a slot past the cache)
 *   nothing is written for row i.
 * kv_new: [n_rows, 576] bf16; slots: [n_rows] int64 (as cp_local_slot
 * returns them); kv_cache: [num_blocks, block_size, 576] bf16, updated in
 * place.  If two rows carry the same slot, one of them is stored, which one
 * is unspecified (cp_local_slot never maps two positions to one slot).
 * Errors: MLA_ERR_INVALID_ARG for null pointers (when n_rows > 0),
 * kv_new or kv_cache not 16-byte aligned, n_rows < 0, num_blocks < 1 or
 * block_size < 1; MLA_ERR_HIP if the launch fails.
 */
int mla_kv_write(const void* kv_new, const int64_t* slots, int64_t n_rows, void* kv_cache,
                 int num_blocks, int block_size, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H_ */
