/*
 * basa.h: C ABI of the MI355X (gfx950) shifted local-window attention library.
 *
 * Source of the operation: "Backend-Agnostic Sparse Attention for Fast High-Resolution
 * Visual Generation" (Ma, Song, Wu, Liu, Zhao; arXiv 2610.08772).
 *   §3.1 "Shifted Window Sparse Attention": the visual token grid is cyclically shifted
 *        by -Delta, partitioned into non-overlapping windows, each window gets standard
 *        scaled dot-product softmax attention, and the outputs are shifted back by +Delta.
 *   App. A.1 "Regular execution with standard attention backends": the partition applies
 *        to grids exactly divisible by the window; windows are independent dense
 *        attention problems.
 *   Fig. 3(b): the operation replaces a DiT's visual self-attention; its inputs are the
 *        already-projected (and position-encoded) q, k, v, its output is the attention
 *        output before the output projection.
 *
 * Conventions shared by every entry point:
 *   - Tensors are contiguous [B, heads, N, head_dim], N = T*H*W tokens flattened
 *     row-major over (t, h, w). q, k, v, out hold the same element type.
 *   - All tensor pointers are DEVICE pointers owned by the caller and must be 16-byte
 *     aligned. The library's own state is the compute-unit count of each device, read on
 *     the first bf16 call there and cached (thread-safe), and the workspaces of split work
 *     items (next item).
 *   - Split work items (bf16 only). The kernel that walks one work item at a time (windows
 *     of 2 or more than 16 key tiles of 64 tokens, the dense baseline, pooled memory,
 *     routed windows, log-sum-exp) splits the items of a last round that would occupy at
 *     most half of the compute units into two halves along the key stream; the half that
 *     finishes second merges them. The halves' partial results go to a workspace of one
 *     (device, stream): for 256 compute units 35.7 MB (128 items x 2 halves x 139,264
 *     bytes, and 4 bytes per item), allocated with hipMalloc, its counters cleared with
 *     hipMemsetAsync on `stream`, on the first call on that stream that splits, and kept
 *     until the process ends; at most 16 per device (calls on further streams run
 *     unsplit). Calls on one stream share it (they run in order); calls on different
 *     streams never do. A stream destroyed while such a call on it still runs
 *     must not be followed, before that call ends, by a new stream with the same handle.
 *     If the allocation fails, or the stream is being captured into a graph and has no
 *     workspace yet, the call runs unsplit (the same result within the bf16 bounds).
 *   - Calls are asynchronous on `stream` (0 = the null stream) and return once the work
 *     is enqueued. Apart from a stream's first split call (above) they allocate, clear and
 *     synchronise nothing, so a sequence of calls can be captured in a HIP graph and
 *     replayed (after a first call on the device, outside the capture, has read its
 *     compute-unit count). Argument errors are reported before any HIP call is made; no
 *     entry point aborts, throws or prints.
 *   - The softmax scale is 1/sqrt(head_dim); softmax statistics are kept in fp32.
 *   - Supported: dtype BASA_DTYPE_F32 or BASA_DTYPE_BF16, head_dim 64 or 128.
 */
#ifndef BASA_H
#define BASA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BASA_DTYPE_F32 = 0,  /* IEEE binary32 */
  BASA_DTYPE_BF16 = 1  /* bfloat16, fp32 accumulation, output rounded to nearest even */
} basa_dtype;

typedef enum {
  BASA_OK = 0,
  BASA_ERR_NULL = 1,        /* a required pointer is NULL */
  BASA_ERR_SHAPE = 2,       /* non-positive size, or window does not divide the grid */
  BASA_ERR_UNSUPPORTED = 3, /* dtype or head_dim outside the supported set */
  BASA_ERR_ALIAS = 4,       /* an output buffer overlaps an input or another output */
  BASA_ERR_OVERFLOW = 5,    /* a size or index does not fit the 32-bit per-head indexing:
                               T*H*W, B*heads and N*head_dim must not exceed 2^31-1, and
                               for bf16 one head must not exceed 0xffffff00 bytes */
  BASA_ERR_HIP = 6,         /* the HIP runtime rejected the launch (hipGetLastError) */
  BASA_ERR_ALIGN = 7,       /* a tensor pointer is not 16-byte aligned */
  BASA_ERR_SCRATCH = 8      /* basa_window_attn_fwd_noalloc: the split work items need more
                               than the static scratch buffer holds (grids of more than 256
                               workgroups; never on MI355X) */
} basa_status;

/*
 * Shifted local-window attention (paper §3.1).
 *
 * Grid (T, H, W) and window (wt, wh, ww): every window size must be positive and divide
 * its grid size exactly (App. A.1); otherwise BASA_ERR_SHAPE. Images use T = wt = 1; the
 * paper's video windows span the whole temporal axis (wt = T), smaller wt is allowed.
 * Shift (st, sh, sw): any integers, reduced modulo (T, H, W). Along each axis, window m
 * local slot l reads and writes the original position (m*w + l + shift) mod n, i.e. the
 * grid is rolled by -shift before partitioning and the output rolled back by +shift.
 * Windows that wrap around the grid edge attend across it; there is no mask.
 *
 * out[b, h, i, :] = sum_{j in win(i)} softmax_j(q_i . k_j / sqrt(head_dim)) v_j.
 *
 * out must not overlap q, k or v (BASA_ERR_ALIAS). Returns a basa_status.
 */
int basa_window_attn_fwd(const void* q, const void* k, const void* v, void* out,
                         int B, int heads, int T, int H, int W,
                         int wt, int wh, int ww, int st, int sh, int sw,
                         int head_dim, int dtype, hipStream_t stream);

/*
 * basa_window_attn_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid it. Same arguments, result and errors,
 * plus BASA_ERR_SCRATCH. It calls no hipMalloc, hipFree or other allocating routine: split
 * work items keep their partial results in a static device array of the library (35.7 MB per
 * device, held until the process ends; room for 128 split items, i.e. grids of up to 256
 * workgroups). Its counters are cleared by a small kernel on `stream` at every call that
 * splits (no memset). Every call on a device uses the same array, so calls that overlap on
 * one device (different streams, or host threads) race; calls in order on one stream do not.
 */
int basa_window_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                 int B, int heads, int T, int H, int W,
                                 int wt, int wh, int ww, int st, int sh, int sw,
                                 int head_dim, int dtype, hipStream_t stream);

/*
 * Dense softmax attention over all N tokens: the baseline the paper's speedups are
 * measured against (§4, Tables 2 and 3, "Dense" rows). It runs the same kernel as
 * basa_window_attn_fwd with grid (1, 1, N), window (1, 1, N) and no shift.
 * Same conventions and errors as basa_window_attn_fwd.
 */
int basa_full_attn_fwd(const void* q, const void* k, const void* v, void* out,
                       int B, int heads, int N, int head_dim, int dtype, hipStream_t stream);

/*
 * K/V pooling for the global memory (paper §3.2 "K/V-Pooled Global Memory", first displayed
 * equation; the count of App. A.1 "Computational complexity"). k, v: [B, heads, T*H*W,
 * head_dim] as for basa_window_attn_fwd. Every frame t is cut into regions of ph x pw
 * tokens starting at (h, w) = (0, 0) of the original (unshifted) grid, gh = ceil(H/ph) by
 * gw = ceil(W/pw) of them; a region cut by the far edge holds only the tokens inside.
 *   kmem[b, h, (t*gh + i)*gw + j, :] = mean of k over region (i, j) of frame t
 * (vmem likewise from v), accumulated in fp32 and stored in dtype (bf16: round to nearest
 * even). kmem, vmem: caller-owned device buffers of B*heads*T*gh*gw*head_dim elements,
 * 16-byte aligned, not overlapping k, v or each other (BASA_ERR_ALIAS).
 * Errors as basa_window_attn_fwd; ph, pw must be positive (BASA_ERR_SHAPE).
 */
int basa_pool_kv(const void* k, const void* v, void* kmem, void* vmem, int B, int heads, int T, int H, int W,
                 int ph, int pw, int head_dim, int dtype, hipStream_t stream);

/*
 * Shifted local-window attention with pooled global memory (paper §3.2, second displayed
 * equation): the queries of every window attend, in one softmax, to the window's own keys
 * and values followed by n_mem memory keys and values shared by all windows of a head:
 *   out[b,h,i,:] = softmax over j in win(i) + memory of (q_i . key_j / sqrt(d)) value_j.
 * kmem, vmem: [B, heads, n_mem, head_dim] device buffers in dtype (for example from
 * basa_pool_kv, n_mem = T*gh*gw); n_mem = 0 with NULL kmem/vmem gives
 * basa_window_attn_fwd's result.
 * lse: optional (NULL = not written) fp32 device buffer [B, heads, N]: the natural-log
 * log-sum-exp of each row's scaled logits, so results over disjoint key sets can be
 * merged as O = (1 - g) O_a + g O_b, g = sigmoid(lse_b - lse_a) (paper App. A.1, last
 * displayed equation). Grid, window, shift, layout and errors as basa_window_attn_fwd;
 * additionally out and lse must not overlap any input or each other (BASA_ERR_ALIAS) and
 * lse must be 4-byte aligned.
 */
int basa_window_attn_mem_fwd(const void* q, const void* k, const void* v, const void* kmem, const void* vmem,
                             int n_mem, void* out, float* lse, int B, int heads, int T, int H, int W, int wt, int wh,
                             int ww, int st, int sh, int sw, int head_dim, int dtype, hipStream_t stream);

/*
 * Window descriptors for true-window routing (paper §3.3 "Content-Adaptive True-Window
 * Routing", its displayed equation): for every window m of the shifted partition,
 *   qbar[b, h, m, :] = mean of q over the window's tokens, kbar likewise from k,
 * accumulated in fp32. qbar, kbar: caller-owned fp32 device buffers [B, heads, n_win,
 * head_dim], n_win = (T/wt)(H/wh)(W/ww), windows numbered as in basa_window_perm, 16-byte
 * aligned, not overlapping q, k or each other. Grid/window/shift, dtype and errors as
 * basa_window_attn_fwd.
 */
int basa_window_means(const void* q, const void* k, float* qbar, float* kbar, int B, int heads, int T, int H,
                      int W, int wt, int wh, int ww, int st, int sh, int sw, int head_dim, int dtype,
                      hipStream_t stream);

/*
 * Top-1 true-window routing (paper §3.3; App. A.2 "Video resolution extrapolation": one
 * routed window, candidates within radius one). For window i of head (b, h):
 *   route[b, h, i] = argmax over candidates j of qbar[b,h,i] . kbar[b,h,j] / sqrt(head_dim)
 * where the candidates are the windows at Chebyshev distance 1 .. radius on the window
 * grid (T/wt, H/wh, W/ww), without wrap-around and never i itself. Ties go to the lowest
 * window index; a window without candidates gets -1. Scores are computed in fp32.
 * qbar, kbar: fp32 device buffers as written by basa_window_means; route: caller-owned
 * int32 device buffer [B, heads, n_win]. Errors: BASA_ERR_NULL, BASA_ERR_SHAPE (grid,
 * window, radius < 0), BASA_ERR_UNSUPPORTED (head_dim), BASA_ERR_ALIGN, BASA_ERR_ALIAS.
 */
int basa_route_top1(const float* qbar, const float* kbar, int32_t* route, int B, int heads, int T, int H, int W,
                    int wt, int wh, int ww, int radius, int head_dim, hipStream_t stream);

/*
 * Shifted window attention with a routed window and pooled memory (paper §3.3: the key
 * and value source of window i is its own tokens, the routed windows' original tokens and
 * the pooled memory). As basa_window_attn_mem_fwd, with route: optional (NULL = none)
 * int32 device buffer [B, heads, n_win] (from basa_route_top1); when route[b, h, i] is a
 * window index, the queries of window i also attend, in the same softmax, to that
 * window's k/v tokens. Entries outside [0, n_win), such as -1, add nothing.
 */
int basa_window_attn_routed_fwd(const void* q, const void* k, const void* v, const int32_t* route,
                                const void* kmem, const void* vmem, int n_mem, void* out, float* lse, int B,
                                int heads, int T, int H, int W, int wt, int wh, int ww, int st, int sh, int sw,
                                int head_dim, int dtype, hipStream_t stream);

/*
 * Window membership export (paper §3.1): perm[m * Wtok + l] = flat original token of
 * local slot l of window m, Wtok = wt*wh*ww, windows numbered row-major over window
 * coordinates (t, h, w) and slots row-major over local coordinates (t, h, w). The table
 * is written on the device by the same index function the attention kernels use.
 * perm: device pointer to T*H*W int32 (4-byte aligned). Same shape and shift rules and
 * errors as basa_window_attn_fwd.
 */
int basa_window_perm(int T, int H, int W, int wt, int wh, int ww, int st, int sh, int sw,
                     int32_t* perm, hipStream_t stream);

/*
 * Interleaved shift schedule (paper §3.1, "Interleaved shift schedule", its three displayed
 * equations). For L sparse-attention layers and window sides (wh, ww), writes the shift of
 * layer l at a denoising step with offset (ch, cw) as (dh[l], dw[l]), l = 0 .. L-1:
 *   per axis, a_i = (i * delta) mod w with delta = max(1, floor(w / L));
 *   b = (a_0, a_K, a_1, a_{K+1}, ...) with K = ceil(L / 2) (the page prints the even-L
 *       pattern; for odd L the first half is one longer);
 *   d[l] = (b_l + c) mod w, c any integer (the page leaves the step offset to the caller).
 * The result is passed as (sh, sw) to basa_window_attn_fwd, with st = 0: the paper's video
 * windows keep the whole temporal axis. dh and dw: HOST arrays of L int32, caller-owned.
 * Host-only: no HIP call. Errors: BASA_ERR_NULL, BASA_ERR_SHAPE (L, wh or ww <= 0).
 */
int basa_shift_schedule(int L, int wh, int ww, int ch, int cw, int32_t* dh, int32_t* dw);

/* Static, NUL-terminated description of a basa_status value. Never NULL. */
const char* basa_status_string(int status);

/* Library ABI version: (major << 16) | minor. */
int basa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BASA_H */
