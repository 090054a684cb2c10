/*
 * attn.h -- C ABI of libattn, scaled dot-product attention forward and
 * backward on AMD Instinct MI355X (gfx950).
 *
 * The operation (one head; every (batch, head) pair is independent, eulerpad
 * "Attention backward" Problem 10 and the [batch, heads, seq, head_dim]
 * layout of the step-by-step derivation's "Forward Pass"):
 *
 *   S = scale * Q K^T            Q: n x d, K: m x d      (mlgrind "Forward")
 *   S_ij = -inf for j > i        only when causal; requires n == m
 *   P = row softmax(S)           stable: the row max is subtracted
 *   O = P V                      V: m x dv, O: n x dv
 *   LSE_i = ln sum_j exp(S_ij)   natural log; P_ij = exp(S_ij - LSE_i)
 *
 * and its gradients for an upstream dO = dL/dO (n x dv)
 * (mlgrind "Backward"; eulerpad Problems 2-6):
 *
 *   dV = P^T dO,  dP = dO V^T,  D_i = rowsum(dO o O)_i = rowsum(dP o P)_i,
 *   dS = P o (dP - D 1^T),  dQ = scale * dS K,  dK = scale * dS^T Q.
 *
 * The backward recomputes P tile by tile from Q, K and LSE (mlgrind "Edge
 * cases and conventions"); it never stores P.  Only the stored-dS dQ mode
 * (ATTN_DQ_STORED_DS below) keeps an n x m matrix, dS, in the workspace.
 *
 * Conventions for every entry point:
 *  - Tensors are device pointers to contiguous row-major [B, H, rows, cols]
 *    arrays: q [B,H,n,d], k [B,H,m,d], v [B,H,m,dv], o and dout [B,H,n,dv],
 *    dq [B,H,n,d], dk [B,H,m,d], dv_out [B,H,m,dv], lse [B,H,n] (float32).
 *  - dtype ATTN_F32: q, k, v, o, dout, dq, dk, dv_out are float32.
 *    dtype ATTN_BF16: they are bfloat16; ATTN_F16: IEEE binary16.  With
 *    either 16-bit type the products run on 16-bit matrix instructions
 *    with float32 accumulation; softmax statistics, LSE and D are float32,
 *    and P and dS are rounded to the input type before their products.
 *  - Supported (d, dv): ATTN_BF16 and ATTN_F16 any multiples of 8 in 8..128
 *    (each is padded with zero columns to 64 or 128 inside the kernels, so
 *    64 and 128 waste no work); ATTN_F32 any d, dv in 1..128.
 *  - The caller owns every buffer.  The library allocates and frees nothing
 *    and never synchronises: work is enqueued on `stream` (a hipStream_t;
 *    NULL is the default stream) and the call returns.
 *  - All validation happens before anything is enqueued; on an error return
 *    nothing was launched and no output was touched.
 *  - Sizes: B, H, n >= 0 (zero means an empty problem: a successful no-op,
 *    except that attn_bwd with n == 0 zero-fills dk and dv_out); m >= 1 (a
 *    softmax over no keys is undefined); d, dv >= 1.
 *  - The library keeps no mutable global state; concurrent calls on
 *    different streams with distinct outputs are safe.
 */
#ifndef LIBATTN_ATTN_H
#define LIBATTN_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, o, dout, dq, dk, dv_out.  lse is always float32. */
enum attn_dtype { ATTN_F32 = 0, ATTN_BF16 = 1, ATTN_F16 = 2 };

/*
 * Mask modes of attn_fwd_ex / attn_bwd_ex.  The pages define the causal mask
 * for n == m only (mlgrind "Forward" and "Inputs"; eulerpad P8), where the
 * two causal modes coincide; for n_b != m_b they are two readings.
 */
enum attn_mask {
    ATTN_MASK_NONE = 0,                /* every key j < m_b is visible */
    ATTN_MASK_CAUSAL = 1,              /* key j visible from row i when j <= i */
    ATTN_MASK_CAUSAL_BOTTOM_RIGHT = 2  /* j <= i + m_b - n_b: the last query row
                                          sees the last key */
};

/*
 * Tensor layouts of attn_fwd_ex / attn_bwd_ex (all of q, k, v, o, dout, dq,
 * dk, dv_out; lse is always [B, H, n]).  ATTN_LAYOUT_BSHD is what a
 * projection X W produces for all heads at once, so no transpose is needed
 * between the projections and attention.
 */
enum attn_layout {
    ATTN_LAYOUT_BHSD = 0,              /* [B, H, seq, dim], each head contiguous */
    ATTN_LAYOUT_BSHD = 1               /* [B, seq, H, dim], the heads of a row adjacent */
};

/* Return codes. */
enum attn_status {
    ATTN_OK = 0,
    ATTN_EINVAL = 1,          /* null pointer, negative size, m < 1, d or dv < 1, non-finite scale */
    ATTN_ECAUSAL_SHAPE = 2,   /* attn_fwd/attn_bwd: causal with n != m (mlgrind "Inputs") */
    ATTN_EUNSUPPORTED = 3,    /* dtype, (d, dv) pair or mask not built, or unknown flag bits */
    ATTN_EWORKSPACE = 4,      /* workspace NULL or smaller than attn_bwd_workspace_bytes() */
    ATTN_EHIP = 5,            /* the HIP runtime refused a launch */
    ATTN_ESCRATCH = 6         /* attn_bwd_ex_noalloc: the problem needs more scratch than
                                 ATTN_NOALLOC_SCRATCH_BYTES */
};

/*
 * attn_bwd flags.  Bits 0-3 choose how dQ = scale * dS K (eulerpad P5) is
 * accumulated; the keys of each row contribute from several workgroups of
 * the dK/dV kernel, which owns a block of 256 keys and walks the queries.
 *
 *  ATTN_DQ_SEPARATE  a second pass per block of query rows recomputes P, dP
 *                    and dS over the keys and sums dS K in registers:
 *                    deterministic, no atomics, about 40% more matrix work.
 *  ATTN_DQ_ATOMIC    the dK/dV kernel also forms dS K for its keys and adds
 *                    it to a float32 accumulator in the workspace with
 *                    atomic adds; a convert pass writes dq.  The key blocks
 *                    before ATTN_DQ_SPLIT(k) (k blocks of 256 keys; 0 = none)
 *                    are summed instead by the separate pass, which then
 *                    initialises the accumulator.  Float32 addition is not
 *                    associative, so dq can differ in its last bits from run
 *                    to run; dk and dv are deterministic in every mode.
 *                    16-bit dtypes only.
 *  ATTN_DQ_STORED_DS the dK/dV kernel also writes the dS it forms (rounded
 *                    to the input type, as the products use it) into the
 *                    workspace, and a third pass forms dQ = scale * dS K
 *                    from it, recomputing nothing: deterministic, the
 *                    matrix work of the formulas alone, at the price of 2
 *                    bytes of workspace per (query, key) pair in visited
 *                    256 x 256 tiles (under the causal mask only the tiles
 *                    on and below the diagonal; see
 *                    attn_bwd_workspace_bytes_ex).  16-bit dtypes; not with
 *                    ATTN_MASK_CAUSAL_BOTTOM_RIGHT unless n == m and both
 *                    length arrays are NULL; one head's tiles at most 2^31
 *                    bytes.  Otherwise ATTN_EUNSUPPORTED.
 *  ATTN_DQ_AUTO      the library's choice for the shapes, from measurements
 *                    on MI355X: the separate pass, which was the fastest
 *                    mode at every shape timed (writing and re-reading dS
 *                    cost more than its recomputation there).
 */
#define ATTN_DQ_SPLIT(k) ((int)(k) << 12) /* k in 0..255, with ATTN_DQ_ATOMIC only */
enum attn_bwd_flags {
    ATTN_DQ_AUTO = 0,
    ATTN_DQ_ATOMIC = 1,
    ATTN_DQ_SEPARATE = 2,
    ATTN_DQ_STORED_DS = 3,
    /* Bits 8-10 restrict which kernels run (0 = all).  They exist so that
       each kernel can be timed on its own; a caller wanting gradients
       leaves them 0.  Later stages read what earlier ones wrote (the
       preprocess before the other two).  A 16-bit call that includes both
       the preprocess and dQ does the preprocess inside the dQ pass, which
       then runs before dK/dV; the results are the same bits either way.
       With ATTN_DQ_ATOMIC the dQ stage is the separate pass over the keys
       before the split plus the convert pass, and only a call with every
       stage yields dq. */
    ATTN_STAGE_PREPROCESS = 1 << 8,   /* D = rowsum(dO o O), LSE rescale */
    ATTN_STAGE_DKDV = 1 << 9,         /* dK and dV */
    ATTN_STAGE_DQ = 1 << 10           /* dQ */
};

/*
 * Forward.  Writes o [B,H,n,dv] (dtype) and lse [B,H,n] (float32, natural
 * log).  scale is the factor on Q K^T; pass 1/sqrt(d) for the usual choice
 * (mlgrind "Forward": d = Q.shape[-1]).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int n, int m, int d, int dv, float scale, int causal,
             int dtype, void* stream);

/*
 * Forward with per-batch lengths and a mask mode (enum attn_mask).
 *
 * seqlens_q and seqlens_k are device arrays of B int32 (4-byte aligned), or
 * NULL for n and m in every batch element.  Batch element b uses query rows
 * i < n_b = seqlens_q[b] and key rows j < m_b = seqlens_k[b] of its n and m
 * rows; the rest is padding, never read.  Lengths outside [0, n] and
 * [0, m] are clamped into them (the library cannot check device values
 * without synchronising).  Padded query rows, and rows that see no key
 * (m_b == 0, or i < n_b - m_b under ATTN_MASK_CAUSAL_BOTTOM_RIGHT), are
 * written as o = 0 and lse = -inf.  No n == m requirement.  layout is an
 * enum attn_layout; with ATTN_LAYOUT_BSHD and a 16-bit dtype,
 * max(n, m) * H * max(d, dv) * 2 must not exceed 2^30 (ATTN_EUNSUPPORTED).
 * Otherwise as attn_fwd, which is attn_fwd_ex with NULL lengths, mask
 * ATTN_MASK_CAUSAL or ATTN_MASK_NONE and ATTN_LAYOUT_BHSD.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                const int* seqlens_q, const int* seqlens_k,
                int B, int H, int n, int m, int d, int dv, float scale, int mask,
                int layout, int dtype, void* stream);

/*
 * Bytes of device workspace attn_bwd_ex needs for these sizes, mask mode
 * (enum attn_mask) and flags (a multiple of 256; zero for an empty problem
 * or invalid arguments).  Holds per-row D and rescaled LSE
 * (2*B*H*round_up(n, 128) floats), plus, in the dQ mode the flags select
 * (16-bit dtypes; ATTN_DQ_AUTO needs nothing more):
 *  - ATTN_DQ_ATOMIC: the float32 dQ accumulator, B*H*round_up(n, 128)*(64
 *    or 128) floats;
 *  - ATTN_DQ_STORED_DS: B*H*t tiles of 256*256 16-bit dS values, with
 *    t = N(N+1)/2 under a causal mask and t = N*M without one,
 *    N = ceil(n/256), M = ceil(m/256).
 */
size_t attn_bwd_workspace_bytes_ex(int B, int H, int n, int m, int d, int dv, int mask,
                                   int dtype, int flags);

/*
 * attn_bwd_workspace_bytes_ex without a mask argument: the largest size
 * over the mask modes, so it suffices for attn_bwd and attn_bwd_ex with any
 * mask.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int n, int m, int d, int dv, int dtype,
                                int flags);

/*
 * Backward.  Inputs q, k, v, o (the forward output), dout and lse (from
 * attn_fwd on the same q, k, v, scale and causal).  Writes dq, dk, dv_out
 * with the shapes of q, k and v.  workspace must be device memory of at
 * least attn_bwd_workspace_bytes() bytes, 256-byte aligned; its contents on
 * entry do not matter.  Output buffers must not overlap inputs.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv_out,
             int B, int H, int n, int m, int d, int dv, float scale, int causal,
             int dtype, int flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward with per-batch lengths and a mask mode, the counterpart of
 * attn_fwd_ex (same lengths, mask, scale; lse from attn_fwd_ex).  Padded
 * query rows and rows that see no key get dq = 0; padded key rows get
 * dk = dv_out = 0.  Workspace size as for attn_bwd (attn_bwd_workspace_bytes
 * with the same B, H, n, m, d, dv, dtype).  Otherwise as attn_bwd.
 */
int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv_out,
                const int* seqlens_q, const int* seqlens_k,
                int B, int H, int n, int m, int d, int dv, float scale, int mask,
                int layout, int dtype, int flags, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * attn_bwd_ex for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument.  The per-row D and rescaled LSE (and, in the
 * atomic dQ mode, the float32 dQ accumulator; in the stored-dS mode the dS
 * tiles) go to a static device array of ATTN_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on each GPU it runs on until the process ends.
 * ATTN_DQ_AUTO runs the separate pass here; a problem whose scratch
 * (attn_bwd_workspace_bytes_ex with that mode) exceeds the array returns
 * ATTN_ESCRATCH before anything is enqueued.  Every call on a GPU shares that GPU's one array and leaves
 * its contents there: calls that overlap on one GPU (different streams or
 * host threads) race and give wrong results, so serialise them.  The first
 * call on each device looks up the array's address (hipGetSymbolAddress,
 * with that device current); no call allocates or frees memory.  Arguments,
 * the current-device rule and the results are otherwise those of
 * attn_bwd_ex.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
int attn_bwd_ex_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv_out,
                        const int* seqlens_q, const int* seqlens_k,
                        int B, int H, int n, int m, int d, int dv, float scale, int mask,
                        int layout, int dtype, int flags, void* stream);

/*
 * Projection gradients of the multi-head self-attention layer around the
 * attention (eulerpad "Attention backward" Problems 7 and 10; datatweets
 * "Step 4").  Tokens are rows, T = B * n; with ATTN_LAYOUT_BSHD the
 * attention tensors [B, n, H, dim] are exactly these [T, H * dim] matrices,
 * so the calls chain without copies:
 *
 *   attn_out_proj_bwd -> do_cat -> attn_bwd_ex (BSHD) -> dq, dk, dv -> attn_in_proj_bwd
 *
 * dtype ATTN_BF16 or ATTN_F16 (16-bit products, float32 accumulation);
 * weight gradients are written in float32, the others in dtype.  Sizes:
 * T >= 0; d_model, hd = H*d and hdv = H*dv multiples of 8, at least 8;
 * every matrix at most 2^30 bytes.  Rows are contiguous (row stride = row
 * length); 16-byte aligned pointers.  Validation and streams as for
 * attn_fwd.  Nothing is allocated.
 *
 * attn_out_proj_bwd: for Y = O_cat W_O with o_cat [T, hdv], w_o
 * [hdv, d_model] and g = dL/dY [T, d_model], writes dw_o = o_cat^T g
 * [hdv, d_model] and do_cat = g w_o^T [T, hdv] (its column block h is head
 * h's dL/dO).
 */
int attn_out_proj_bwd(const void* o_cat, const void* g, const void* w_o, float* dw_o,
                      void* do_cat, int T, int d_model, int hdv, int dtype, void* stream);

/*
 * attn_in_proj_bwd: for Q = X W_Q, K = X W_K, V = X W_V with x [T, d_model],
 * w_q, w_k [d_model, hd], w_v [d_model, hdv] and the attention gradients
 * dq_cat, dk_cat [T, hd], dv_cat [T, hdv], writes dw_q = x^T dq_cat,
 * dw_k = x^T dk_cat ([d_model, hd]), dw_v = x^T dv_cat ([d_model, hdv]) and
 * dx = dq_cat w_q^T + dk_cat w_k^T + dv_cat w_v^T ([T, d_model]).
 */
int attn_in_proj_bwd(const void* x, const void* w_q, const void* w_k, const void* w_v,
                     const void* dq_cat, const void* dk_cat, const void* dv_cat, float* dw_q,
                     float* dw_k, float* dw_v, void* dx, int T, int d_model, int hd, int hdv,
                     int dtype, void* stream);

/* Static string naming a status code. */
const char* attn_status_str(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_ATTN_H */
