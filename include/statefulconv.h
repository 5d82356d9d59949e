/*
 * statefulconv.h — C ABI of the MI355X (gfx950) stateful causal short
 * convolution library (libstatefulconv.so).
 *
 * The operation: a per-channel (depthwise) causal conv1d over variable-length
 * token batches, optionally dilated, with bias and SiLU, whose per-request
 * history of the last (width-1)*dilation raw inputs lives in a slot-indexed
 * state pool; plus the CCA variant (depthwise then per-head grouped conv, a
 * residual mix and a one-token-delayed value).
 *
 * Defining passages (page title, section):
 *  - "vllm.model_executor.layers.mamba.ops.cpu.gdn_attention":
 *    _spec_aware_nonspec (decode conv update, then varlen prefill conv with
 *    query_start_loc / cache_indices / has_initial_state, bias, SiLU),
 *    _conv_buffer_view (state as (num_slots, dim, state_len)),
 *    cpu_gdn_attention_core (zero tokens is a no-op; state_len vs width-1).
 *  - "vllm.models.qwen4_exp.nvidia.ple_layer", Qwen4ExpPLELayer:
 *    conv_state_len = (kernel-1)*dilation, dilated depthwise Conv1d,
 *    _short_conv (state capacity check, weights cast to the input dtype),
 *    _short_conv_dilated_dispatch (decode call, then prefill call, then the
 *    prefill checkpoint export), get_kv_cache_spec (checkpoint grid >= state
 *    length, so a checkpoint window holds inputs only).
 *  - "vllm.model_executor.models.zaya", ZayaCCA: the two Conv1d modules,
 *    project (residual mix, output layout) and _mix_with_state (decodes first,
 *    then prefills; history masked by has-state; new history = last n inputs;
 *    delayed value shifted by one token).
 *
 * Conventions for every entry point:
 *  - Pointers marked (device) are device pointers; (host) are host pointers,
 *    read during the call only. The library never allocates or frees device
 *    memory: the caller owns every buffer.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *    is the default stream). No call synchronises with the host or reads
 *    device memory from the host, so calls may be captured in a HIP graph.
 *  - Arguments are validated on the host before any launch; an error status
 *    means nothing was launched. A launch failure returns SC_ERR_HIP.
 *  - Device-side metadata is trusted but never dereferenced out of bounds:
 *    a slot outside [0, num_slots) is a padding row (zero history, no state
 *    read or write); token rows are clamped to [0, num_tokens).
 *  - Documented, unchecked preconditions (checking needs a host sync):
 *    query_start_loc is non-decreasing with first entry 0 and last entry
 *    num_tokens; slots (and checkpoint slots) are distinct within one call;
 *    `out` does not overlap `x` (exact aliasing is rejected).
 *  - Zero tokens or zero requests: SC_OK, nothing launched; descriptor and
 *    size arguments are still validated, but no pointer is required then
 *    (empty tensors may carry NULL data pointers).
 */
#ifndef STATEFULCONV_H
#define STATEFULCONV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SC_ABI_VERSION 3

typedef enum {
  SC_OK = 0,
  SC_ERR_NULL_ARG = -1,        /* a required pointer is NULL */
  SC_ERR_INVALID_ARG = -2,     /* a size, stride, enum or grid is out of range */
  SC_ERR_DTYPE = -3,           /* dtype not supported by this entry point */
  SC_ERR_STATE_CAPACITY = -4,  /* state_len < (width-1)*dilation */
  SC_ERR_UNSUPPORTED = -5,     /* valid but not built here (e.g. width > 8) */
  SC_ERR_HIP = -6              /* the HIP runtime reported a launch error */
} sc_status;

typedef enum { SC_DTYPE_F32 = 0, SC_DTYPE_BF16 = 1 } sc_dtype;
typedef enum { SC_ACT_NONE = 0, SC_ACT_SILU = 1 } sc_activation;
/* State pool layout (GDN and PLE pages, `is_conv_state_dim_first`): DS =
 * (num_slots, C, S), a channel's entries adjacent (GDN `_conv_buffer_view`);
 * SD = (num_slots, S, C), the cache viewed transposed. Entries are oldest
 * first in both. */
typedef enum { SC_STATE_DS = 0, SC_STATE_SD = 1 } sc_state_layout;

/* Depthwise conv descriptor (host struct, read during the call only).
 * x, out, weight, bias and the state pool share `dtype` (the PLE layer casts
 * its weights to the input dtype); accumulation is fp32. */
typedef struct {
  int32_t channels;       /* C >= 1 */
  int32_t width;          /* K in [1, 8] */
  int32_t dilation;       /* d >= 1 */
  int32_t state_len;      /* S, entries per channel of a state row; S < H = (K-1)*d
                             -> SC_ERR_STATE_CAPACITY; S > 2^20 -> SC_ERR_INVALID_ARG.
                             S > H is a buffer sized for speculative rollback
                             (GDN page, _spec_forward: width-1 + num_spec); the
                             non-speculative calls keep their window in entries
                             [0, H) of each row and leave [H, S) untouched (GDN
                             page, _spec_aware_nonspec, first width-1 columns). */
  int32_t dtype;          /* sc_dtype */
  int32_t activation;     /* sc_activation */
  int64_t x_row_stride;   /* elements between token rows of x, >= C */
  int64_t out_row_stride; /* elements between token rows of out, >= C */
  int64_t state_indices_stride; /* >= 1; row stride of a 2-D index tensor whose
                                   column 0 holds the slot */
  int32_t state_layout;   /* sc_state_layout of every state pool the call touches */
} sc_conv_desc;

/* Prefill checkpoint export (optional). For prefill request r, the m-th
 * checkpoint (m = 1 .. cu_ckpt[r+1]-cu_ckpt[r], and m*grid <= L_r) writes the
 * state window ending at token offset p = m*grid of this chunk — the raw inputs
 * x_r[p-H .. p) — into pool slot ckpt_slots[cu_ckpt[r] + m - 1]. */
typedef struct {
  int32_t grid;              /* g; 0 = no export; else g >= H required */
  const int32_t* cu_ckpt;    /* (device) B+1 exclusive prefix of checkpoint counts */
  const int32_t* ckpt_slots; /* (device) destination slots, flat; NULL (an empty
                                array: no request reaches a checkpoint) exports
                                nothing */
} sc_ckpt_desc;

/* Residual fusion and row mapping, optional on every depthwise call (PLE page
 * "vllm.models.qwen4_exp.nvidia.ple_layer", _short_conv: the conv result is
 * accumulated into `residual`, optionally adding `outer_residual` in the same
 * pass; the dispatch's token_indices let the calls address the speculative and
 * non-speculative rows of a mixed batch in place). NULL = plain call
 * (out = conv). With a descriptor, logical row j of the call (the row the
 * plain call would use) lives at physical row
 *   p = token_indices ? token_indices[j] : j
 * of x, out and outer_residual, and the stored value is, in fp32,
 *   out[p] = (accumulate ? out[p] : 0) + conv_j (+ outer_residual[p])
 * with one final rounding (the additions follow the conv's activation).
 *   token_indices     (device) int32 per logical row, or NULL; entries must be
 *                     distinct rows in [0, num_physical_rows) (an entry outside
 *                     is clamped: no memory fault, that row's results unspecified)
 *   num_physical_rows rows of x / out / outer_residual; required with token_indices
 *   accumulate        0 or 1: out holds the residual on entry (read, then written)
 *   outer_residual    (device) rows like out, or NULL; must not alias out
 *   outer_row_stride  elements between its rows (>= C) */
typedef struct {
  const int32_t* token_indices;
  int64_t num_physical_rows;
  int32_t accumulate;
  const void* outer_residual;
  int64_t outer_row_stride;
} sc_conv_fuse;

/* Varlen prefill: for request r (token rows [qsl[r], qsl[r+1]) of x), slot
 * s = state_indices[r*stride], flag h = has_initial_state[r]:
 *   ext = [h ? pool[s][c][0 .. H) : zeros (oldest first), x_r]
 *   out[t, c] = act(bias[c] + sum_k weight[c, k] * ext[c, H + t - (K-1-k)*d])
 *   pool[s][c][0 .. H) = last H entries of ext (bit-exact copies)
 * A zero-length request produces nothing and leaves its slot untouched.
 *   x                 (device) (num_tokens, C) rows of x_row_stride elements
 *   out               (device) (num_tokens, C) rows of out_row_stride
 *   weight            (device) (C, K) row-major
 *   bias              (device) (C) or NULL
 *   state_pool        (device) (num_slots, C, S) contiguous
 *   query_start_loc   (device) int32 (batch+1)
 *   state_indices     (device) int32, entry r at r*state_indices_stride
 *   has_initial_state (device) uint8 (batch), required (the PLE page raises
 *                     without it)
 *   ckpt              (host) NULL or a checkpoint descriptor */
sc_status sc_conv_prefill_varlen(const sc_conv_desc* desc, const void* x, void* out,
                                 const void* weight, const void* bias,
                                 void* state_pool, int32_t num_slots,
                                 const int32_t* query_start_loc,
                                 const int32_t* state_indices,
                                 const uint8_t* has_initial_state, int32_t batch,
                                 int64_t num_tokens, const sc_ckpt_desc* ckpt,
                                 const sc_conv_fuse* fuse, void* stream);

/* Decode / multi-token update: `batch` requests of exactly q tokens each,
 * request r owning rows [r*q, (r+1)*q) of x (x viewed as (batch, q, C)), all q
 * tokens consumed. Same arithmetic and state rule as the prefill call.
 *   has_initial_state (device) uint8 (batch) or NULL = every request continues
 *                     its saved state (decodes always do). */
sc_status sc_conv_update(const sc_conv_desc* desc, const void* x, void* out,
                         const void* weight, const void* bias, void* state_pool,
                         int32_t num_slots, const int32_t* state_indices,
                         const uint8_t* has_initial_state, int32_t batch,
                         int32_t q, const sc_conv_fuse* fuse, void* stream);

/* Speculative multi-token update on a rolling buffer (GDN page
 * "vllm.model_executor.layers.mamba.ops.cpu.gdn_attention", _spec_forward,
 * per-sequence rolling buffer; PLE page "vllm.models.qwen4_exp.nvidia.ple_layer",
 * ple_conv mode "spec" with num_accepted_tokens and spec_query_len).
 * `batch` requests of exactly q tokens (request r owns rows [r*q, (r+1)*q)),
 * pool rows of S = desc->state_len >= H entries. With slot s and
 *   a = num_accepted_tokens[r] clamped to [1, min(q, S-H+1)]
 * (the range in which the page's slices are well formed; values outside it
 * act as the nearest bound):
 *   ext      = [pool[s][c][a-1 .. a-1+H), x_r]
 *   out[t,c] = act(bias[c] + sum_k weight[c,k] * ext[c, H + t - (K-1-k)*d])
 *   pool[s]  = [pool[s][c][a .. a+S-q), x_r]   (length S, bit-exact copies)
 * A slot outside [0, num_slots) is a padding row: zero history, no write.
 * q > S -> SC_ERR_INVALID_ARG (the drafts would not fit the buffer).
 *   num_accepted_tokens (device) int32 (batch), required.
 * Other arguments as for sc_conv_update (no has_initial_state: speculative
 * requests always continue their buffer). */
sc_status sc_conv_update_spec(const sc_conv_desc* desc, const void* x, void* out,
                              const void* weight, const void* bias, void* state_pool,
                              int32_t num_slots, const int32_t* state_indices,
                              const int32_t* num_accepted_tokens, int32_t batch,
                              int32_t q, const sc_conv_fuse* fuse, void* stream);

/* Speculative update with a draft count per request (GDN page
 * "vllm.model_executor.layers.mamba.ops.cpu.gdn_attention", _spec_forward,
 * the per-sequence loop over spec_query_start_loc that serves batches whose
 * requests draft different numbers of tokens). Request r owns rows
 * [query_start_loc[r], query_start_loc[r+1]) of x and out; with
 * q_r = query_start_loc[r+1] - query_start_loc[r], the rule of
 * sc_conv_update_spec applies to it with q = q_r (a clamped to
 * [1, min(q_r, S-H+1)]). A request with q_r = 0 is skipped (the page's loop
 * continues past it): nothing is read or written for it.
 *   query_start_loc (device) int32 (batch+1), non-decreasing,
 *                   query_start_loc[0] >= 0, query_start_loc[batch] <= num_tokens.
 *   max_query_len   (host) a bound on every q_r; must be <= S
 *                   (SC_ERR_INVALID_ARG otherwise). A request that breaks
 *                   the bound, or whose rows leave [0, num_tokens), is
 *                   skipped whole (its rows and slot are left as they were).
 *   num_tokens      (host) rows of x and out.
 * Other arguments as for sc_conv_update_spec. batch = 0, num_tokens = 0 or
 * max_query_len = 0: no-op. */
sc_status sc_conv_update_spec_varlen(const sc_conv_desc* desc, const void* x, void* out,
                                     const void* weight, const void* bias, void* state_pool,
                                     int32_t num_slots, const int32_t* state_indices,
                                     const int32_t* num_accepted_tokens,
                                     const int32_t* query_start_loc, int32_t batch,
                                     int64_t num_tokens, int32_t max_query_len,
                                     const sc_conv_fuse* fuse, void* stream);

/* Row copies between a slot pool and a dense buffer; each row is row_bytes.
 * They are the state gather and write-back of "vllm.model_executor.models.zaya",
 * ZayaCCA._mix_with_state, on their own: that method reads each request's
 * history as the pool row its slot index names, masked to zeros when the
 * request has no initial state, and afterwards writes the new history back to
 * the same row; the GDN page ("vllm.model_executor.layers.mamba.ops.cpu.
 * gdn_attention", _spec_forward) indexes its conv-state cache by slot in the
 * same way. Byte copies, so bit-exact for any dtype and either layout.
 * gather: dense[i] = pool[idx[i*idx_stride]], or zeros when that index is
 *         outside [0, num_slots) (a padding row has no history).
 * scatter: pool[idx[i*idx_stride]] = dense[i]; out-of-range indices skipped;
 *          two equal in-range indices race (a documented precondition:
 *          distinct indices, as sc_validate_metadata checks).
 *   pool, dense, idx (device, caller-owned); n rows; row_bytes >= 1.
 * Errors: NULL pointer with n > 0 -> SC_ERR_NULL_ARG; negative n or
 * num_slots, row_bytes < 1 or idx_stride < 1 -> SC_ERR_INVALID_ARG;
 * launch failure -> SC_ERR_HIP. n = 0: no-op. Asynchronous on `stream`. */
sc_status sc_state_gather(const void* pool, int32_t num_slots, int64_t row_bytes,
                          const int32_t* idx, int64_t idx_stride, int32_t n,
                          void* dense, void* stream);
sc_status sc_state_scatter(const void* dense, int64_t row_bytes,
                           const int32_t* idx, int64_t idx_stride, int32_t n,
                           void* pool, int32_t num_slots, void* stream);

/* CCA q/k conv descriptor (host struct). bf16 only (SC_ERR_DTYPE otherwise). */
typedef struct {
  int32_t num_q_heads;    /* nq */
  int32_t num_kv_heads;   /* nkv; nq % nkv == 0 */
  int32_t head_dim;       /* hd */
  int32_t t0;             /* depthwise kernel size */
  int32_t t1;             /* grouped kernel size */
  int32_t dtype;          /* SC_DTYPE_BF16 */
  int64_t q_row_stride, k_row_stride, v_cur_row_stride, v_del_row_stride;
  int64_t out_row_stride;
  int64_t decode_slot_stride, prefill_slot_stride;
} sc_cca_desc;

/* CCA q/k conv with per-request state (ZayaCCA.project + _mix_with_state).
 * Tokens: num_decodes one-token decode rows first (always continuing their
 * state), then prefill rows with offsets prefill_qsl (rebased to 0).
 * With C = (nq+nkv)*hd raw channels [q | k] and n = t0+t1-2:
 *   dw   = depthwise conv (t0 taps, bias) of [history, raw], materialised in
 *          bf16: summed in fp32 from the bias (hd = 128, t1 = 2: taps in
 *          pairs on the two-term bf16 dot product; other shapes: a fused
 *          multiply-add chain in tap order) and rounded to bf16, which is the
 *          exact value rounded once except where the fp32 sum's own rounding
 *          moves it across a bf16 midpoint (a few values in 10^7 on normally
 *          distributed data)
 *   yg   = grouped conv (nq+nkv groups of hd, t1 taps, bias) of dw, fp32 acc.
 *   out row = [yg_q + 0.5(q + k of the head's kv group) |
 *              yg_k + mean over the group's q heads of that residual |
 *              v_cur | previous token's v_del (first token: saved delayed
 *              value if it has state, else delayed_init, NULL = zeros)]
 *   conv_state[s] = last n raw inputs; delayed_state[s] = last v_del row.
 *   q (T, nq*hd), k (T, nkv*hd), v_cur, v_del (T, nkv*hd/2), out
 *   (T, (nq+2*nkv)*hd); w_dw (C, t0), b_dw (C), w_gr (C, hd, t1), b_gr (C),
 *   delayed_init (nkv*hd/2) or NULL; conv_state (num_slots, C, n; may be NULL
 *   when n = 0),
 *   delayed_state (num_slots, nkv*hd/2); slot arrays int32, has-state uint8.
 *   All (device). num_tokens must equal num_decodes + prefill_qsl[last]. */
sc_status sc_cca_qk_conv(const sc_cca_desc* desc, const void* q, const void* k,
                         const void* v_cur, const void* v_del, void* out,
                         const void* w_dw, const void* b_dw, const void* w_gr,
                         const void* b_gr, const void* delayed_init,
                         void* conv_state, void* delayed_state, int32_t num_slots,
                         int32_t num_decodes, const int32_t* decode_slots,
                         int32_t num_prefills, const int32_t* prefill_qsl,
                         const int32_t* prefill_slots,
                         const uint8_t* prefill_has_initial_state,
                         int64_t num_tokens, void* stream);

/* Checks the device-side preconditions the calls above document but cannot
 * check without a host sync (a debugging and test aid, not for the hot path):
 * waits for `stream`, copies the metadata to the host and returns
 * SC_ERR_INVALID_ARG if
 *   query_start_loc (device, batch+1, or NULL to skip) is not non-decreasing
 *                   from query_start_loc[0] = 0 to query_start_loc[batch] = num_tokens;
 *   state_indices   (device, batch rows of idx_stride, or NULL to skip) has an
 *                   entry >= num_slots, or two equal non-negative entries
 *                   (negative entries are padding rows);
 * else SC_OK. It allocates no device memory and launches nothing. batch = 0:
 * SC_OK without touching the pointers; a HIP error while copying: SC_ERR_HIP;
 * negative sizes, idx_stride < 1, or arrays too large to copy to the host:
 * SC_ERR_INVALID_ARG. */
sc_status sc_validate_metadata(const int32_t* query_start_loc, const int32_t* state_indices,
                               int64_t idx_stride, int32_t batch, int64_t num_tokens,
                               int32_t num_slots, void* stream);

/* Static string for a status code. */
const char* sc_status_string(sc_status status);

/* SC_ABI_VERSION of the built library. */
int32_t sc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* STATEFULCONV_H */
