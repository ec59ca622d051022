/*
 * librelpos -- attention with a decomposed relative-position bias, for AMD
 * Instinct MI355X (gfx950).  C ABI: plain pointers, sizes and status codes.
 *
 * The operation (prhub summary page of vllm-project/vllm PR #55629, "DeepEncoder
 * relative-position attention fused into a Triton kernel", section 关键源码片段,
 * the RelPosAttention.forward branch):
 *
 *   tokens       i = qh*W + qw over an H x W grid, N = H*W (row-major flattening
 *                of a [B, H, W, C] activation);
 *   rel_h[i,kh]  = sum_c q[i,c] * rel_pos_h[qh - kh + H - 1, c]   (unscaled q)
 *   rel_w[i,kw]  = sum_c q[i,c] * rel_pos_w[qw - kw + W - 1, c]
 *   out[i,:]     = sum_j softmax_j( scale * q_i . k_j + rel_h[i, j/W] + rel_w[i, j%W] ) v[j,:]
 *
 * The page shows add_decomposed_rel_pos only as a call; the table index
 * qh - kh + H - 1 (resp. qw - kw + W - 1) is the reading this library takes.
 * The dense [B, heads, N, N] bias of the unfused path is never formed: the
 * attention kernel streams K/V tiles with an online softmax (the page's
 * implementation section, item 1) and adds the two bias terms per tile.
 *
 * Conventions shared by every call:
 *   - All tensors are dense, row-major, 16-byte aligned, and live in device
 *     memory of the current HIP device (hipSetDevice).  The caller allocates and
 *     owns every buffer; the library allocates nothing at run time, keeps no
 *     state besides a per-device cache of device properties and the fixed
 *     scratch array of relpos_attn_fused_noalloc (RELPOS_SCRATCH_BYTES per
 *     device, reserved when the library's device code is loaded), and never
 *     synchronises the host.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL means the null stream)
 *     and completes asynchronously.  Calls are safe from several host threads.
 *   - Checks run in this order, and the first failure is returned: sizes
 *     (E_SHAPE), dtypes (E_DTYPE), scalars (E_VALUE); then, unless B*heads == 0
 *     (an OK no-op), NULL pointers (E_NULL), alignment (E_ALIGN), overlap of an
 *     output with any other operand (E_ALIAS), and finally that every pointer is
 *     device memory of the current device whose allocation holds the whole
 *     operand (E_DEVICE; a too-short allocation is E_SHAPE).
 *   - On any validation failure nothing is launched and the status says why.
 *     No call prints or throws.
 */
#ifndef RELPOS_H_
#define RELPOS_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RELPOS_ABI_VERSION 4

typedef enum relpos_dtype {
  RELPOS_BF16 = 0,
  RELPOS_FP16 = 1,
  RELPOS_FP32 = 2
} relpos_dtype;

typedef enum relpos_status {
  RELPOS_OK = 0,
  RELPOS_E_NULL = 1,    /* a required pointer is NULL */
  RELPOS_E_SHAPE = 2,   /* a size is out of range (D != 64, H or W < 1, too large, ...) */
  RELPOS_E_DTYPE = 3,   /* unsupported dtype or dtype combination */
  RELPOS_E_ALIGN = 4,   /* a pointer is not 16-byte aligned */
  RELPOS_E_DEVICE = 5,  /* a pointer is not device memory of the current device */
  RELPOS_E_ALIAS = 6,   /* an output overlaps an input or the other output */
  RELPOS_E_LAUNCH = 7,  /* the kernel launch failed (HIP error) */
  RELPOS_E_HIP = 8,     /* another HIP runtime call failed */
  RELPOS_E_VALUE = 9    /* a scalar argument is invalid (e.g. a non-finite scale) */
} relpos_status;

/*
 * relpos_build: the per-query bias tables of the decomposed relative position.
 *
 * Defines (PR #55629 page, key source snippet, add_decomposed_rel_pos call):
 *   rel_h[b,h,i,kh] = sum_c q[b,h,i,c] * rel_pos_h[i/W - kh + H - 1, c]
 *   rel_w[b,h,i,kw] = sum_c q[b,h,i,c] * rel_pos_w[i%W - kw + W - 1, c]
 * with bf16/fp16 products accumulated in fp32 and stored as fp32.
 *
 * Arguments (device pointers unless said otherwise):
 *   q          [B, heads, H*W, D]   in_dtype  (the unscaled queries)
 *   rel_pos_h  [2H-1, D]            in_dtype
 *   rel_pos_w  [2W-1, D]            in_dtype
 *   rel_h      [B, heads, H*W, H]   fp32, written
 *   rel_w      [B, heads, H*W, W]   fp32, written
 *   B, heads   >= 0, B*heads <= 65535 (B*heads == 0 is an OK no-op; pointers are then not read)
 *   H, W       >= 1, H*W <= 2^24, H <= 4096, W <= 4096
 *   D          must be 64
 *   in_dtype   RELPOS_BF16 or RELPOS_FP16
 *   stream     hipStream_t to enqueue on
 * Errors: E_SHAPE, E_DTYPE, E_NULL, E_ALIGN, E_DEVICE, E_ALIAS (rel_h/rel_w
 * overlapping each other or an input), E_LAUNCH.
 */
relpos_status relpos_build(const void* q, const void* rel_pos_h, const void* rel_pos_w,
                           float* rel_h, float* rel_w,
                           int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                           relpos_dtype in_dtype, void* stream);

/*
 * relpos_attn_fwd: attention over all N = H*W keys with the decomposed bias.
 *
 * Defines (PR #55629 page, key source snippet, the SDPA fallback it replaces):
 *   out[b,h,i,:] = sum_j P[i,j] v[b,h,j,:],
 *   P[i,:] = softmax_j( scale * q[b,h,i,:] . k[b,h,j,:]
 *                       + rel_h[b,h,i, j/W] + rel_w[b,h,i, j%W] ).
 * Computed without the dense bias: K/V are streamed through LDS in tiles of
 * the key grid, scores go through an exp2-based online softmax with fp32
 * accumulators, and Q.K^T and P.V run on bf16/fp16 MFMA.
 *
 * Arguments (device pointers):
 *   q, k, v    [B, heads, H*W, D]   in_dtype
 *   rel_h      [B, heads, H*W, H]   fp32 (as written by relpos_build)
 *   rel_w      [B, heads, H*W, W]   fp32
 *   out        [B, heads, H*W, D]   out_dtype, written; must not overlap any input
 *   B, heads   >= 0, B*heads <= 65535 (B*heads == 0 is an OK no-op)
 *   H, W       >= 1, H*W <= 2^24, H <= 4096, W <= 4096, and
 *              B*heads*ceil(H*W/64) < 2^31
 *   D          must be 64
 *   scale      multiplies q.k only (not the bias); any sign.  It must be 0
 *              or satisfy 2^-64 <= |scale| < inf, else E_VALUE (the kernel
 *              adds rel_w / scale to the q.k accumulator; scale == 0 is
 *              computed exactly as the bias alone)
 *   in_dtype   RELPOS_BF16 or RELPOS_FP16
 *   out_dtype  RELPOS_FP32, or equal to in_dtype
 *   stream     hipStream_t to enqueue on
 * Precision of P.V (fp32 accumulation throughout): for bf16 inputs on grids
 * of N >= 2048 keys where configuration 6 runs (relpos_attn_config), P is
 * rounded to bf16 and v used as is; otherwise P is rounded to fp16 and bf16 v
 * is converted to fp16 when staged.  Rounding P to bf16 adds an error that
 * averages over the keys (mean |error| 3.5e-5 at 64x64, 2.3e-5 at 96x96 on
 * N(0,1) inputs, against 4e-6 with fp16 P).
 * Value range: where bf16 v is converted to fp16, |v| must stay below 65520
 * (larger values become inf and the outputs they reach are not finite), and
 * |v| < 2^-24 is flushed to zero (absolute error below 2^-25).  fp16 v, and
 * bf16 v with bf16 P, are used as is.  Nothing checks the range.
 * Errors: E_SHAPE, E_DTYPE, E_VALUE, E_NULL, E_ALIGN, E_DEVICE, E_ALIAS, E_LAUNCH.
 */
relpos_status relpos_attn_fwd(const void* q, const void* k, const void* v,
                              const float* rel_h, const float* rel_w, void* out,
                              int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                              float scale, relpos_dtype in_dtype, relpos_dtype out_dtype,
                              void* stream);

/*
 * relpos_attn_fwd_ws: relpos_attn_fwd with a caller-provided workspace, which
 * lets the launch split the key range of query units across workgroups.
 *
 * Same operation, arguments, result tolerance and errors as relpos_attn_fwd,
 * plus:
 *   workspace        device memory, 16-byte aligned, not overlapping any
 *                    other operand.  Scratch: its contents on entry are not
 *                    read, and on return it holds partial results.  Calls
 *                    that use one workspace must not run concurrently (on one
 *                    stream they never do).
 *   workspace_bytes  its size; >= relpos_attn_workspace_bytes(...) for the
 *                    current device, else E_SHAPE when the split is chosen.
 *                    When that value is 0 the workspace is not used and may
 *                    be NULL.  A negative size is E_VALUE.
 * Split launch (chosen by the cost model of relpos_attn_config when it is
 * faster): a grid of one 8-wave workgroup per compute unit (P of them) over
 * units of 256 consecutive queries of one (b, h), T key tiles each.  The
 * first floor(units / P) * P units run whole, one round at a time; the rest
 * of the last round are cut at key tile s = (T*k + 6*(k-1))/(k+1) (k =
 * ceil(rest / (P - rest)), rounded to nearest): their heads [0, s) run on
 * `rest` workgroups and their tails [s, T) on the others, k per workgroup;
 * s balances s + 6 against k*(T - s + 6), 6 tiles being the measured fixed
 * cost of one segment.  Heads and tails store their normalised output
 * (fp16), reference maximum and row sum in the workspace, and a second
 * kernel on the same stream merges each unit's head and tail (in that order)
 * and writes its output.  Results are bitwise reproducible run to run, and
 * differ from the unsplit launch by rounding only.
 * Check order: as relpos_attn_fwd up to overlap, then the configuration is
 * chosen (a device query); if it splits, the workspace is checked (NULL,
 * alignment, size, overlap), and finally every pointer, the workspace
 * included, must be device memory of the current device.
 */
relpos_status relpos_attn_fwd_ws(const void* q, const void* k, const void* v,
                                 const float* rel_h, const float* rel_w, void* out,
                                 int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                                 float scale, relpos_dtype in_dtype, relpos_dtype out_dtype,
                                 void* workspace, int64_t workspace_bytes, void* stream);

/*
 * relpos_attn_workspace_bytes: bytes of workspace relpos_attn_fwd_ws needs for
 * this problem on a device with `cu_count` compute units: 0 when the split
 * launch would not be chosen, -1 if a size or the dtype is out of range or
 * cu_count < 1.  Host-only.  The size is cu_count * 2 * (256*64 + 2*256) * 4
 * bytes: two piece slots per workgroup.
 */
int64_t relpos_attn_workspace_bytes(int64_t B, int64_t heads, int64_t H, int64_t W,
                                    relpos_dtype in_dtype, int cu_count);

/*
 * relpos_attn_fused: relpos_build followed by relpos_attn_fwd in one call,
 * without the rel_h / rel_w tensors (the fusion the PR #55629 page's
 * implementation section leaves to the model helper: there rel_h and rel_w are
 * built by add_decomposed_rel_pos before the fused kernel is called).
 *
 * Defines the same `out` as relpos_build + relpos_attn_fwd on the same inputs
 * (same tolerance against the definition; results differ from the two-call
 * path by rounding only).  Three launch forms, chosen by the grid:
 *   - H <= 32, W <= 32 and at most four key tiles of 4 grid rows x 16
 *     columns (ceil(H/4) * ceil(W/16) <= 4; the 14 x 14 windows of windowed
 *     attention, 16 x 16, 8 x 32): the 16-query kernel of configuration 3,
 *     whose workgroup of 64 queries first forms their bias rows on MFMA
 *     (fp32 accumulation) into LDS, 64*(H + W) floats beside the K/V
 *     staging, and reads them from there in the key loop.  No workspace: the
 *     workspace argument is not read and may be NULL with workspace_bytes 0.
 *   - bf16 inputs with W % 32 == 0, H % 4 == 0, H*W >= 2048 and at least 6
 *     blocks of 32 queries per (b, h): the 12-wave kernel of configuration 6
 *     on a persistent grid of min(units, CUs) workgroups (units =
 *     ceil(B*heads*H*W/32 / 6)).  For each unit a workgroup first computes its
 *     6 blocks' bias rows on MFMA (fp32 accumulation, the same products as
 *     relpos_build, so the result equals the two-call path's bit for bit),
 *     then runs the key loop reading them back.  With H, W <= 64 the tables
 *     are staged once per workgroup in LDS, a unit inside one head keeps its
 *     rows in LDS, and only a unit spanning two heads (or a partial last
 *     unit) puts them in its workspace slot, one slot per b*heads; on larger
 *     grids every workgroup uses its own slot.  No second kernel.
 *   - otherwise: each workgroup of the persistent split launch of
 *     relpos_attn_fwd_ws (one 8-wave workgroup per compute unit, merge kernel
 *     when split) computes the bias rows of its 256 queries and reads them
 *     back per key tile: rel_w rows from its slot of the workspace, rel_h rows
 *     from LDS when 256*(roundup(H,4)+4) floats fit beside the K/V staging
 *     (H <= 72 on a 160 KB LDS), else from the slot as well; a fixed cost of
 *     12 tiles per segment in place of 6; the last round is left whole when
 *     its split would not be faster (max(s + 12, k*(T - s + 12)) + 4 >= T + 12).
 *
 * Arguments: q, k, v, out, B, heads, H, W, D, scale, in_dtype, out_dtype and
 * stream as for relpos_attn_fwd (with the same scale rule and bf16 v range),
 * plus
 *   rel_pos_h  [2H-1, D]  in_dtype (device)
 *   rel_pos_w  [2W-1, D]  in_dtype (device)
 *   workspace  device scratch, 16-byte aligned, not overlapping any other
 *              operand; contents on entry are not read.  Calls sharing a
 *              workspace must not run concurrently.  Not read, and not
 *              checked, on the small grids of the first form.
 *   workspace_bytes  >= relpos_fused_workspace_bytes(...) for the current
 *              device (else E_SHAPE); negative is E_VALUE.
 * Errors: E_SHAPE, E_DTYPE, E_VALUE, E_NULL, E_ALIGN, E_ALIAS (out or the
 * workspace overlapping another operand), E_DEVICE, E_HIP (device query),
 * E_LAUNCH.  Check order: sizes, dtypes, scalars; then (B*heads > 0) NULL and
 * alignment of all seven pointers (six on the small grids of the first
 * form), out overlapping an input; then the device's compute-unit count is
 * queried, and the workspace size (E_SHAPE), workspace overlap and device
 * memory of every operand are checked.
 */
relpos_status relpos_attn_fused(const void* q, const void* k, const void* v,
                                const void* rel_pos_h, const void* rel_pos_w, void* out,
                                int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                                float scale, relpos_dtype in_dtype, relpos_dtype out_dtype,
                                void* workspace, int64_t workspace_bytes, void* stream);

/* Size of the per-device scratch array behind relpos_attn_fused_noalloc. */
#define RELPOS_SCRATCH_BYTES (96u << 20)

/*
 * relpos_attn_fused_noalloc: relpos_attn_fused for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * serving loops that forbid allocation).  The workspace is a fixed array of
 * RELPOS_SCRATCH_BYTES (96 MiB) of device memory per device, held by the
 * library from the load of its device code to the end of the process; the
 * call itself allocates nothing.
 *
 * Same operation, arguments (without workspace and workspace_bytes), result
 * and errors as relpos_attn_fused, plus
 *   E_SHAPE  when relpos_fused_workspace_bytes(...) for the current device
 *            exceeds RELPOS_SCRATCH_BYTES (on 256 compute units, for any
 *            batch: with the 12-wave kernel when H + W > 512, otherwise when
 *            roundup(H, 4) + roundup(W, 16) > 252; 64x64, 48x80 and 96x96
 *            fit).
 *   E_HIP    when the scratch array's address cannot be looked up.
 * The scratch contents are never read before they are written within a call,
 * so nothing needs clearing between calls.  Every call on one device shares
 * that device's array: calls on one stream are ordered, but calls that can
 * overlap on one device (several streams, several host threads) race and must
 * not be issued.
 */
relpos_status relpos_attn_fused_noalloc(const void* q, const void* k, const void* v,
                                        const void* rel_pos_h, const void* rel_pos_w, void* out,
                                        int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                                        float scale, relpos_dtype in_dtype, relpos_dtype out_dtype,
                                        void* stream);

/*
 * relpos_fused_workspace_bytes: workspace bytes relpos_attn_fused needs on a
 * device with `cu_count` compute units.  0 on the small grids of the first
 * form above (H, W <= 32, ceil(H/4) * ceil(W/16) <= 4).  With the 12-wave
 * kernel (the second form): slots * 6 * 32 * (H + W) * 4 with slots =
 * min(units, cu_count) (one slot of bias rows per workgroup), or, when H, W
 * <= 64, min(B*heads, units, cu_count) (only the units spanning two heads or
 * partial use a slot): 1.2 MB at 64x64 with 12 heads, against 25.2 MB of
 * rel_h / rel_w; one slot per workgroup is at most the size of rel_h / rel_w
 * once B*heads*H*W/192 >= cu_count.  Otherwise:
 *   cu_count * (2 * (256*64 + 2*256) + 256 * (roundup(H, 4) + roundup(W, 16))) * 4
 * (two split pieces and one slot of bias rows per workgroup).  -1 if a size
 * or the dtype is out of range or cu_count < 1.  Host-only.
 */
int64_t relpos_fused_workspace_bytes(int64_t B, int64_t heads, int64_t H, int64_t W,
                                     relpos_dtype in_dtype, int cu_count);

/*
 * relpos_attn_config: the launch configuration relpos_attn_fwd (with_workspace
 * = 0) or relpos_attn_fwd_ws (with_workspace != 0) uses for a problem on a
 * device with `cu_count` compute units.  Host-only: it launches nothing and
 * touches no device, so it can be called anywhere.
 *
 *   0: workgroups of 8 waves x 32 queries, one workgroup per compute unit;
 *      a workgroup's two waves per SIMD share one K/V staging.
 *   1: workgroups of 4 waves x 32 queries, two per compute unit.
 *   3: workgroups of 4 waves x 16 queries (16x16x32 MFMA), chosen when a
 *      unit has at most 4 key tiles of 4 x 16 grid cells (ceil(H/4) *
 *      ceil(W/16) <= 4), where its shorter pipeline is measured fastest.
 *   5: configuration 0 with the key range split over one workgroup per
 *      compute unit (relpos_attn_fwd_ws only).
 *   6: workgroups of 12 waves over 6 blocks of 32 queries, one workgroup per
 *      compute unit; the two waves of a block take the even and the odd key
 *      tiles and merge at the end, and a workgroup may cover the last blocks
 *      of one (b, h) and the first of the next.  Needs N >= 192 and the full
 *      160 KB LDS.  Considered for bf16 inputs with N >= 2048 (where its P.V
 *      runs in bf16), at 0.75 * 1.05 of a configuration-0 round per round of
 *      ceil(B*heads*ceil(N/32)/6) workgroups.
 *
 * Otherwise the choice compares times in workgroup rounds (one round = one 4-wave
 * workgroup per SIMD pair of every compute unit running all T key tiles of
 * its queries): configuration 0 counts every started round of its
 * workgroups as a full one, at 0.91 of a configuration-1 round for bf16
 * inputs (whose V conversion it shares) and 0.985 for fp16 (which needs none;
 * both measured); configuration 1 counts a last round with at most one
 * workgroup per compute unit at 0.77 (a lone workgroup runs one wave per
 * SIMD, measured faster per tile); configuration 5 costs the 8-wave factor
 * times 1.06 (the persistent grid's measured per-tile overhead) times (full
 * rounds + (max(s + 6, k*(T - s + 6)) + 4) / T) in the terms of
 * relpos_attn_fwd_ws, and is considered only with a workspace, a last round
 * to split and k <= 4.  Ties go to the lower number.
 * Returns -1 if a size or the dtype is out of range (as relpos_attn_fwd
 * checks them) or cu_count < 1.
 */
int relpos_attn_config(int64_t B, int64_t heads, int64_t H, int64_t W, relpos_dtype in_dtype,
                       int cu_count, int with_workspace);

/*
 * relpos_attn_fwd_cfg: relpos_attn_fwd_ws in a launch configuration chosen by
 * the caller instead of relpos_attn_config's model, for measuring and testing
 * the configurations against each other.
 *
 * Same operation, arguments, tolerance and errors as relpos_attn_fwd_ws, plus
 *   config  one of the configurations listed with relpos_attn_config, or -1
 *           for the automatic choice (then exactly relpos_attn_fwd_ws).  Any
 *           other value is E_VALUE; a configuration whose LDS does not fit the
 *           device is E_SHAPE.  Configuration 5 needs the workspace
 *           relpos_attn_workspace_bytes reports for a split problem (E_NULL
 *           without one, E_SHAPE if too small); the others ignore it.
 */
relpos_status relpos_attn_fwd_cfg(const void* q, const void* k, const void* v,
                                  const float* rel_h, const float* rel_w, void* out,
                                  int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                                  float scale, relpos_dtype in_dtype, relpos_dtype out_dtype,
                                  int config, void* workspace, int64_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* relpos_status_string(relpos_status s);

/* RELPOS_ABI_VERSION of the built library. */
int relpos_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RELPOS_H_ */
