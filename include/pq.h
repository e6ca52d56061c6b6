/*
 * pq.h — C ABI of the PARO W4A8 linear hot path for AMD Instinct MI355X (gfx950).
 *
 * The method is the one on the page "ParoQuant (PARO) W4A8 on gfx1201 — engineering log"
 * (sections "Format" and "Design"): activations are channel-scaled and rotated through 8
 * layers of pairwise Givens rotations local to each 128-channel group, quantised per
 * (token, group) to OCP e4m3 with code-domain row-sums (the prologue), then multiplied by
 * AWQ-packed uint4 asymmetric group-128 weights whose zero point enters as a row-sum
 * correction (the GEMM). Merged linears carry up to 3 activation partitions.
 *
 * Conventions for every entry point:
 *  - Pointers named *_d are device pointers, *_h host pointers. The caller allocates every
 *    buffer and keeps it alive until the stream has passed the call; the library allocates
 *    nothing and keeps no pointer after returning.
 *  - Work is queued on `stream` (a hipStream_t; NULL = the default stream). Nothing
 *    synchronises. Asynchronous device faults surface at the caller's next synchronisation.
 *  - Every argument is validated before anything is launched. On error nothing is launched,
 *    no output is touched, a negative PQ_ERR_* code is returned and pq_last_error() holds a
 *    message (per calling thread). M == 0 is a valid no-op.
 *  - Element types: f16 and bf16 are passed as uint16_t bit patterns.
 *  - No environment variables are read and nothing is printed.
 */
#ifndef PQ_H_
#define PQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PQ_ABI_VERSION 1
#define PQ_GROUP 128
#define PQ_LAYERS 8
#define PQ_MAX_PARTITIONS 3
/* "no boundary" value for pb1 / pb2 */
#define PQ_NO_BOUNDARY 0x7FFFFFFF

typedef struct ihipStream_t* pq_stream_t; /* same type as hipStream_t */

enum pq_status {
  PQ_OK = 0,
  PQ_ERR_NULL = -1,      /* a required pointer is NULL */
  PQ_ERR_SHAPE = -2,     /* a size or stride is out of range */
  PQ_ERR_ALIGN = -3,     /* a pointer or stride is not aligned as required */
  PQ_ERR_PARTITION = -4, /* P or the partition boundaries are inconsistent */
  PQ_ERR_RECORDS = -5,   /* a 128-slice of `pairs` is not a permutation of 0..127 */
  PQ_ERR_WORKSPACE = -6, /* workspace smaller than pq_gemm_workspace_bytes() */
  PQ_ERR_DEVICE = -7     /* the HIP runtime reported an error at launch */
};

/* ABI version of the loaded library (PQ_ABI_VERSION it was built with). */
int pq_abi_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* pq_last_error(void);

/*
 * Rotation records (host only, load time).
 *
 * pairs_h  int16 [8, K]: per layer, every 128-slice is a permutation of 0..127; pair q of
 *          layer r is (pairs[r, 2q], pairs[r, 2q+1]), channels local to group q/64.
 * theta_h  f16 [8, K/2]: the angle of pair q of layer r.
 * rec_h    out, 8 * (K/2) records of 8 bytes, layout [8][K/2]; within each (layer, group) the
 *          64 records are stored in the order the prologue's 64 lanes consume them. Record of
 *          layer r, lane l: uint32 w, f16 f1, f16 f2, where w holds the lane's pair as it
 *          computes it, u = w & 0x7F (first operand) and v = (w >> 8) & 0x7F (second), bit 7
 *          "v arrives negated" (t = -1; layers 1..7), bit 15 "the output kept in registers is
 *          v's", bits 16-23 the LDS hand-off row the lane reads v from (layers 1..7), bits 24-31
 *          the row it writes its other output to (layers 0..6). With c/s = f16
 *          round-to-nearest-even of the fp64 cos/sin of the f16 angle for the pair listed as
 *          (u, v) (listing it as (v, u) negates sin), (f1, f2) = (c, t*s) when u's output is kept
 *          and (-s, t*c) when v's is. The lane reads w = t*v and computes keep = f1*u + f2*w, the
 *          kept output bit for bit, and hand = f1*w - f2*u, the other output times t (negated
 *          once more when v's output is kept), which the reading lane's t accounts for. Layer 0
 *          reads u and v from the quad image (t = 1); layer 7 keeps u's output and writes both to
 *          the image, v's as t*hand. In between each lane's kept output is the next layer's u.
 *          For P partitions call once per partition and concatenate: [P][8][K/2].
 * Source: section "Format" (pairs/theta) and "Design" item 3 (8-byte records).
 * Errors: PQ_ERR_NULL, PQ_ERR_SHAPE (K <= 0 or K % 128), PQ_ERR_RECORDS.
 */
int pq_build_records(const int16_t* pairs_h, const uint16_t* theta_h, int K, void* rec_h);

/*
 * Partition plan (host only, load time). A merged linear stacks J projections along N (in this
 * order), each with its own rotation (pairs, theta, channel scales). Adjacent projections whose
 * rotation data are bytewise identical merge into one partition, so the GEMM's limit of 3 applies
 * to runs of distinct rotations, as the loader on the pages does for qwen3_5's in_proj_qkvz (q, k
 * and v share one rotation: 4 projections, 2 partitions).
 * Source: "Design" item 4 (partition select, adjacent identical rotations merged into runs) and
 * "Traps hit" (the 3-partition limit is on distinct rotations).
 *
 * J        number of projections, 1..64.
 * ncols_h  int [J]: columns of each projection, positive multiples of 16.
 * pairs_h, theta_h, cs_h   J pointers each: int16 [8, K], f16 [8, K/2], f16 [K] (host).
 * P_out    out: number of partitions (1..3).
 * pb_out   out int [2]: pb1, pb2 for pq_gemm (PQ_NO_BOUNDARY when unused).
 * rep_out  out int [3]: for each partition, the first projection of its run (-1 when unused);
 *          its rotation data go into pq_build_records / the prologue's cs for that partition.
 * Errors: PQ_ERR_NULL, PQ_ERR_SHAPE, PQ_ERR_PARTITION (more than 3 runs, or a run boundary that
 *         is not a multiple of 128 columns). Outputs are untouched on error.
 */
int pq_plan_partitions(int J, const int* ncols_h, const int16_t* const* pairs_h,
                       const uint16_t* const* theta_h, const uint16_t* const* cs_h, int K,
                       int* P_out, int* pb_out, int* rep_out);

/*
 * Weight packing (device, load time): AWQ tensors -> the GEMM's operands.
 *
 * qweight_d int32 [K, N/8], qzeros_d int32 [K/128, N/8]: AWQ words, nibble i of word j holds
 *           column 8j + (0,2,4,6,1,3,5,7)[i]; zero points stored as-is (section "Format").
 * scales_d  f16 [K/128, N].
 * wpk_d     out, pq_packed_weight_bytes(K, N) bytes: first K*N/2 bytes hold the same 4-bit
 *           codes reordered into matrix-core fragment order (1 KiB per 16 columns x 128-group,
 *           each 16-column strip's groups contiguous);
 *           then, per 16 columns, ceil(3*(K/128)/32) KiB of bf16 operands for the zero-point
 *           epilogue (the f32 values 8*sc + fl16(sc*(zp-8)) split into two bf16 pieces);
 *           then (K/128) * N f32 column factors 512*sc for the prefill fold.
 *           Returns 0 for shapes the library rejects.
 * sz_d      out, f16 [K/128, N, 2]: {sc, fl16(sc * (zp - 8))} interleaved ("Design" item 1).
 * Requires K % 128 == 0, N % 16 == 0, 16-byte aligned wpk_d, 4-byte aligned others.
 */
size_t pq_packed_weight_bytes(int K, int N);
int pq_pack_weights(const int32_t* qweight_d, const int32_t* qzeros_d, const uint16_t* scales_d,
                    int K, int N, void* wpk_d, uint16_t* sz_d, pq_stream_t stream);

/*
 * Rotate-quant prologue (device): per partition p, token m, group g —
 *   v = x * cs_p; 8 Givens layers (a, b) -> (c*a + s*b, c*b - s*a) in fp32 without fused
 *   multiply-add; amax = max|v|; asg = amax * fl32(1/448); codes = e4m3(v * fl32(1/asg))
 *   (OCP E4M3FN, round to nearest even, NaN -> 0, -0 -> +0, clamped to +-448);
 *   rs = fl32(exact sum of the decoded codes). An all-zero group gives codes 0, asg 0, rs 0.
 * Source: "Format" (inference identity), "Design" items 2-3, "Gates passed" (amax*(1/448.f)).
 *
 * x_d    f16 [M, ldx] (first K columns used), 4-byte aligned, ldx even and >= K.
 * rec_d  [P][8][K/2] records from pq_build_records, 8-byte aligned.
 * cs_d   f16 [P, K] pre-inverted channel scales (multiply), 4-byte aligned.
 * a_d    out u8 [P, M, K] e4m3 codes, 16-byte aligned.
 * asg_d  out f32 [P, M, K/128] group scales; rs_d out f32 [P, M, K/128] code-domain sums.
 * 1 <= P <= 3, K % 128 == 0.
 */
int pq_rotate_quant(const uint16_t* x_d, int64_t ldx, int M, int K, int P, const void* rec_d,
                    const uint16_t* cs_d, uint8_t* a_d, float* asg_d, float* rs_d,
                    pq_stream_t stream);

/*
 * W4A8 group GEMM (device): for column n in partition p(n) = [n >= pb1] + [n >= pb2],
 *   y[m, n] = bf16_rne( sum_g asg_p[m,g] * ( sc[g,n] * sum_{k in g} D(A_p[m,k]) * (c[k,n] - 8)
 *                                            - fl16(sc[g,n]*(zp[g,n]-8)) * rs_p[m,g] ) )
 * i.e. the zero point enters as a row-sum correction ("Design" item 1), one launch for all
 * partitions ("Design" item 4). Rows m >= M of y are never written.
 *
 * a_d/asg_d/rs_d  prologue outputs for P partitions (layouts above), a_d 16-byte aligned.
 * wpk_d, sz_d     from pq_pack_weights for this K, N.
 * pb1, pb2        partition boundaries: PQ_NO_BOUNDARY (or >= N) when unused; finite ones
 *                 satisfy 0 < pb1 < pb2 < N and are multiples of 128; P must equal
 *                 1 + the number of boundaries below N.
 * y_d             out bf16 [M, ldy], ldy >= N, 4-byte aligned, ldy even.
 * ws_d, ws_bytes  device workspace of at least pq_gemm_workspace_bytes(M, N, K) bytes, 16-byte
 *                 aligned (may be NULL when that is 0: M <= 16). For M > 16 the call first
 *                 writes the activation operand of the zero-point epilogue and a transposed
 *                 copy of asg there (sized for up to 3 partitions); its contents need no
 *                 initialisation and are not kept.
 * Requires K % 128 == 0, N % 16 == 0.
 */
size_t pq_gemm_workspace_bytes(int M, int N, int K);
int pq_gemm(const uint8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
            const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
            int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream);

/*
 * The prologue and the GEMM sharing the GEMM's workspace, so that nothing runs between them
 * (the producer writes the consumer's operand layout directly: "2026-09-08 (late): fused TILED
 * prologue for prefill"; the zero-point operand is the one of "2026-09-12: zero-point epilogue").
 *
 * pq_rotate_quant_for_gemm: pq_rotate_quant (same arguments, outputs and results) that, when
 *   M > 16, also writes into ws_d what pq_gemm would otherwise derive from ASG and RS at the
 *   start of each call: the activation-side zero-point operand and the group scales transposed,
 *   computed with the same arithmetic. ws_d/ws_bytes: as for pq_gemm (at least
 *   pq_gemm_workspace_bytes(M, N, K) bytes, 16-byte aligned); unused when M <= 16.
 * pq_gemm_prepared: pq_gemm (same arguments and results) that reads those operands from ws_d
 *   instead of writing them. ws_d must hold what pq_rotate_quant_for_gemm wrote for this same
 *   (a_d, asg_d, rs_d, M, K, P), with nothing written to ws_d in between; the library cannot
 *   check this, and any other contents give wrong outputs (never an out-of-bounds access: every
 *   offset follows from the validated M, K and P). For M <= 16 it is pq_gemm.
 */
int pq_rotate_quant_for_gemm(const uint16_t* x_d, int64_t ldx, int M, int K, int P, const void* rec_d,
                             const uint16_t* cs_d, uint8_t* a_d, float* asg_d, float* rs_d, void* ws_d,
                             size_t ws_bytes, pq_stream_t stream);
int pq_gemm_prepared(const uint8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
                     const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
                     int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream);

/*
 * pq_gemm without a workspace, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments, arithmetic,
 * kernels and results as pq_gemm, minus ws_d/ws_bytes: at M > 16 the zero-point operand and the
 * transposed group scales go to a scratch array the library holds on each device (16 MiB, from
 * the first call on that device until the process ends), sized for the call's own P:
 *   P * ceil(M/16) * ceil(3*(K/128)/32) KiB  +  P * (K/128) * M * 4 bytes (rounded up to 256),
 * e.g. M = 8192 at K = 17408 for P = 1, or M = 2048 at K = 5120 for P = 3. Larger calls return
 * PQ_ERR_SHAPE before anything is launched. Nothing is allocated; no initialisation is needed
 * (every byte read is written earlier in the same call). All calls on one device share its
 * scratch, so calls that overlap on a device (several streams or threads) race; serialise them.
 * pq_gemm_noalloc_max_scratch_bytes returns the scratch size.
 */
size_t pq_gemm_noalloc_max_scratch_bytes(void);
int pq_gemm_noalloc(const uint8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
                    const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
                    int64_t ldy, pq_stream_t stream);

/*
 * Per-token activation-scale path (device): the same rotation, one e4m3 scale per
 * (partition, token) instead of per (token, group) -
 *   amax = max over the whole row of |v|; as = amax * fl32(1/448); codes = e4m3(v * fl32(1/as))
 *   (same encoder as pq_rotate_quant); rs[g] = fl32(exact sum of the decoded codes of group g).
 *   An all-zero row gives codes 0, as 0, rs 0.
 * Source: "Numbers" (the per-token prefill: token scale = the largest group scale, plain
 * row-sums, the scale applied in the GEMM epilogue), "2026-09-08: MXFP4-PARO prod decode" item 1
 * (fused prologue, row kept on chip), "2026-09-09 (late)" (plain row-sums, no bf16 scratch row).
 *
 * pq_rotate_quant_tok: arguments as pq_rotate_quant, but as_d out f32 [P, M] token scales and
 *   K <= 18432 (the rotated row is kept on chip: 16 waves x 9 groups).
 * pq_gemm_tok: arguments as pq_gemm with as_d = AS [P, M] in place of ASG:
 *   y[m, n] = bf16_rne( as_p[m] * sum_g ( sc[g,n] * sum_{k in g} D(A_p[m,k]) * (c[k,n] - 8)
 *                                         - fl16(sc[g,n]*(zp[g,n]-8)) * rs_p[m,g] ) )
 *   The workspace (pq_gemm_tok_workspace_bytes) is needed at every M > 0; no initialisation.
 */
int pq_rotate_quant_tok(const uint16_t* x_d, int64_t ldx, int M, int K, int P, const void* rec_d,
                        const uint16_t* cs_d, uint8_t* a_d, float* as_d, float* rs_d,
                        pq_stream_t stream);
size_t pq_gemm_tok_workspace_bytes(int M, int N, int K);
int pq_gemm_tok(const uint8_t* a_d, const float* as_d, const float* rs_d, int M, int K, int P,
                const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
                int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream);

/*
 * Per-group int8 activation mode (device): the same rotation and per-(token, group) scales with
 * int8 codes -
 *   amax = max over the group of |v|; asg = fl32(amax / 127); codes = clamp(round-half-even(
 *   fl32(v * fl32(1/asg))), -127, 127); rs = the integer sum of the group's codes (as f32).
 *   An all-zero group gives codes 0, asg 0, rs 0.
 * pq_gemm_i8: arguments as pq_gemm with int8 codes; the same formula with D(A) replaced by the
 *   integer code (products on the integer matrix core, exact in int32 per group).
 * Source: "2026-09-11: I8 mode -- int8 activations on the iu8 WMMA" (scale amax/127, round and
 * clamp to +-127, integer row-sums, integer products, the e4m3 path's fold algebra and SZ),
 * "2026-09-11 (evening): per-group int8 on the A-tiled band" (per-group granularity).
 * pq_rotate_quant_i8: arguments as pq_rotate_quant; a_d out int8 [P, M, K], 16-byte aligned.
 */
int pq_rotate_quant_i8(const uint16_t* x_d, int64_t ldx, int M, int K, int P, const void* rec_d,
                       const uint16_t* cs_d, int8_t* a_d, float* asg_d, float* rs_d,
                       pq_stream_t stream);
int pq_gemm_i8(const int8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
               const void* wpk_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
               int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream);

/*
 * int5 bit-plane weights (W5A8): 5-bit asymmetric codes c in 0..31 per 128-group with zero points
 * in 0..31 and f16 scales, W = sc * (c - zp); the activations and the GEMM are those of
 * pq_rotate_quant / pq_gemm. The matrix core takes c - 16, exact in e4m3 for every code.
 * Source: "2026-09-10: int5 W5A8 ParoQuant -- round-to-nearest checkpoint, kernel and first
 * served numbers" (the "int5-bitplane" checkpoint: the low four bits in the int4 AWQ words, the
 * fifth bits in [K, N/32] int32 planes; the int4 path's algebra and zero-point fold carry over).
 *
 * pq_pack_weights5 (device, load time):
 *   qweight_d int32 [K, N/8], qzeros_d int32 [K/128, N/8]: the codes' and zero points' low four
 *             bits in the AWQ layout of pq_pack_weights.
 *   qweight_hi_d int32 [K, N/32], qzeros_hi_d int32 [K/128, N/32]: fifth bits; bit j of word w
 *             is column 32w + j.
 *   scales_d  f16 [K/128, N].
 *   wpk5_d    out, pq_packed_weight5_bytes(K, N) bytes: the K*N/2-byte nibble image of
 *             pq_pack_weights, then K*N/8 bytes of fifth bits in fragment order (256 bytes per
 *             16 columns x 128-group: lane l's 32-bit word carries the bits of its 32 codes),
 *             then the zero-point epilogue operand built from sc * (zp - 16), then the f32 column
 *             factors 512*sc as in pq_pack_weights.
 *   sz_d      out, f16 [K/128, N, 2]: {sc, fl16(sc * (zp - 16))}.
 *   Requires K % 128 == 0, N % 32 == 0, 16-byte aligned wpk5_d, 4-byte aligned others. Returns
 *   0 bytes from pq_packed_weight5_bytes for shapes the library rejects.
 * pq_gemm5: arguments as pq_gemm with wpk5_d/sz_d from pq_pack_weights5 (N % 32 == 0):
 *   y[m, n] = bf16_rne( sum_g asg_p[m,g] * ( sc[g,n] * sum_{k in g} D(A_p[m,k]) * (c[k,n] - 16)
 *                                            - fl16(sc[g,n]*(zp[g,n]-16)) * rs_p[m,g] ) )
 *   Same workspace as pq_gemm (pq_gemm_workspace_bytes); at M > 16 the prefill tiles are 256x256
 *   on a ring of two stages (128x128 when a partition boundary is off a 256-column line).
 */
size_t pq_packed_weight5_bytes(int K, int N);
int pq_pack_weights5(const int32_t* qweight_d, const int32_t* qweight_hi_d, const int32_t* qzeros_d,
                     const int32_t* qzeros_hi_d, const uint16_t* scales_d, int K, int N, void* wpk5_d,
                     uint16_t* sz_d, pq_stream_t stream);
int pq_gemm5(const uint8_t* a_d, const float* asg_d, const float* rs_d, int M, int K, int P,
             const void* wpk5_d, const uint16_t* sz_d, int N, int pb1, int pb2, uint16_t* y_d,
             int64_t ldy, void* ws_d, size_t ws_bytes, pq_stream_t stream);

/*
 * Fused producer (device): residual add + RMSNorm + the per-group rotate-quant, one launch.
 * Source: "2026-09-02/03: rotation stream (fused add + RMSNorm + rotate + quant producers)"
 * (one kernel per norm-fed linear returning the normalised row, the new residual and A/ASG/RS;
 * the residual exact, the normalised row within ppm of a CPU reference). Per token row:
 *   h = fl16(f32(x) + f32(res));                       the new residual, written to res_out
 *   hs = fl16((h * rstd) * w'),  rstd = 1 / sqrt(mean_k(h^2) + eps),  w' = 1 + w (gemma != 0)
 *        or w (gemma == 0), all in binary32 (the row's sum of squares in a fixed order)
 *   A, ASG, RS = pq_rotate_quant of hs (same arithmetic, every partition).
 *
 * x_d, res_d  f16 [M, ldx] / [M, ldr] (first K columns used); res_out_d f16 [M, ldo]: either
 *             disjoint from res_d's rows, or res_d itself with ldo == ldr (in place; the launch
 *             then keeps one workgroup per 4 tokens, which at M <= 64 is slower than the split form
 *             a separate res_out gets). Any other overlap returns PQ_ERR_SHAPE. No other output
 *             may overlap an input. w_d f16 [K].
 * hs_d        out f16 [M, K] contiguous.
 * rec_d, cs_d, a_d, asg_d, rs_d  as pq_rotate_quant.
 * eps > 0 and finite; 1 <= P <= 3; K % 128 == 0 and K <= 18432 (each row is kept on chip);
 * x_d, res_d, res_out_d, w_d, hs_d 16-byte aligned, ldx, ldr, ldo multiples of 8 and >= K.
 */
int pq_add_rms_rotate_quant(const uint16_t* x_d, int64_t ldx, const uint16_t* res_d, int64_t ldr,
                            const uint16_t* w_d, float eps, int gemma, int M, int K, int P,
                            const void* rec_d, const uint16_t* cs_d, uint16_t* res_out_d, int64_t ldo,
                            uint16_t* hs_d, uint8_t* a_d, float* asg_d, float* rs_d, pq_stream_t stream);

/*
 * Verification hooks: run the exact device arithmetic the prologue uses on plain arrays, so
 * tests can check it exhaustively.
 *  pq_e4m3_encode: codes_d[i] = E(q_d[i]) with the prologue's encoder (n >= 0).
 *  pq_recip_f32:   y_d[i] = 1 / x_d[i] with the prologue's reciprocal.
 *  pq_bf16_round:  out_d[i] = the bf16 bits of x_d[i] with the rounding of the GEMM outputs and the
 *                  zero-point operands (round to nearest even; a NaN becomes a quiet NaN with its
 *                  sign and top payload bits), pairs through the epilogues' packed convert.
 * Arguments: device arrays of n elements (n >= 0; 4-byte aligned floats, 2-byte aligned outputs).
 * Errors: PQ_ERR_SHAPE (n < 0 or too large), PQ_ERR_NULL, PQ_ERR_ALIGN, PQ_ERR_DEVICE.
 */
int pq_e4m3_encode(const float* q_d, uint8_t* codes_d, int64_t n, pq_stream_t stream);
int pq_recip_f32(const float* x_d, float* y_d, int64_t n, pq_stream_t stream);
int pq_bf16_round(const float* x_d, uint16_t* out_d, int64_t n, pq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PQ_H_ */
