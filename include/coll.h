/*
 * coll.h - collective communication primitives over p logical ranks whose
 * buffers all live in one MI355X's HBM.
 *
 * Each call carries all p ranks at once: rank r is index r of the pointer
 * arrays, so the communicator of the pages reduces to (p, ordered pointer
 * arrays) and rank order is array order.  Semantics follow
 *   [A] "集合通信：原语、算法、NCCL 实现与拓扑映射" (llm-infra-atlas, hpc/04):
 *       notation p, [n], elementwise + in {sum,min,max} (chapter preamble);
 *       primitive table (section 0); sections 1.1-1.6; ring all-reduce 2.2;
 *       bus-bandwidth factors 2.5.
 *   [B] "Collective Communication：AllReduce、AllGather、ReduceScatter 与
 *       All-to-All" (charlestar.github.io): ragged All-to-All; CUDA-stream
 *       semantics ("API return is not completion"); in-place offset rules;
 *       failure semantics (a collective is not a transaction).
 *   [C] "详解分布式训练8大集合通信原语：从Send/Recv到All2All"
 *       (bjdmk.com.cn): Scatter (section 3.3), Gather (section 4.3).
 *
 * Common contract
 * ---------------
 * - Arguments typed `const void* const*` / `void* const*` are HOST arrays
 *   of length p holding DEVICE pointers; index = rank.  The caller owns
 *   every device buffer; the library neither allocates nor frees them.
 * - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *   validates on the host and enqueues kernels; it returns before the work
 *   is done.  Results may be read after the stream is synchronised or
 *   after an event recorded on it has completed ([B], CUDA Stream).
 * - Validation is synchronous and complete before anything is enqueued; a
 *   call that returns an error has enqueued nothing.  n == 0 is a no-op
 *   returning COLL_OK (pointers are then not inspected).
 * - Every device pointer must be aligned to its element size (else
 *   COLL_ERR_INVALID_ARG); buffers that share one 16-byte misalignment take
 *   the 16-byte vector path, others an element-wide path.
 * - Aliasing: the output ranges must be pairwise disjoint and may not
 *   overlap any input range, except the in-place forms listed with each
 *   call ([B], In-place).  Input ranges may overlap each other.  A
 *   violation returns COLL_ERR_ALIAS.
 * - Errors are not transactional ([B], failure semantics): if the device
 *   faults mid-call, outputs may be partially written.
 * - Calls that run concurrently on different streams over the same buffers
 *   race; ordering is the caller's (stream order or events).
 * - Thread safety: every entry point may be called from several host
 *   threads, except coll_finalize, which must not run concurrently with
 *   any other call.
 * - Work balancing: large calls hand part of their tiles (or token rows)
 *   to workgroups through counters in a static device array, one slot of
 *   eight counters per stream (assigned on first use, up to 1024 streams
 *   per device; later streams and hipStreamPerThread deal out all their
 *   work in turn instead).  Each launch leaves its counters at zero when
 *   it completes, so the calls of one stream, which run in order, share a
 *   slot; nothing is allocated for it.  Results do not depend on how the
 *   work was handed out.
 */
#ifndef COLL_H_
#define COLL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  bf16 is reduced in fp32 and narrowed once with
 * round-to-nearest-even.  COLL_U8 is raw bytes (e.g. FP8 payloads): the
 * data-movement calls (Broadcast, AllGather, Gather, Scatter, All-to-All,
 * Alltoallv, coll_moe_pack) accept it; the reductions and the combine
 * return COLL_ERR_INVALID_ARG for it. */
typedef enum { COLL_F32 = 0, COLL_BF16 = 1, COLL_I32 = 2, COLL_U8 = 3 } coll_dtype_t;

/* Elementwise reduction ([A] preamble: + is sum, min or max).
 * COLL_AVG: the sum in the schedule's order, then divided by p ([A] 1.4:
 * older NCCL had no average, callers summed and divided by the world
 * size): one IEEE fp32 division (bf16 narrowed after it), and for int32 C
 * division of the wrapped sum, truncating toward zero. */
typedef enum { COLL_SUM = 0, COLL_MIN = 1, COLL_MAX = 2, COLL_AVG = 3 } coll_op_t;

typedef enum {
  COLL_OK = 0,
  COLL_ERR_INVALID_ARG = 1,  /* bad p, null pointer, bad enum, root out of range, size overflow */
  COLL_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement */
  COLL_ERR_ALIAS = 3,        /* illegal overlap between buffers */
  COLL_ERR_HIP = 4           /* the HIP runtime reported an error; see coll_last_hip_error */
} coll_status_t;

/* AllReduce schedules ([A] 2.2 ring; 2.3 recursive doubling and
 * halving-doubling).  On one device every schedule reads each input once
 * and writes each output once; they differ in the floating-point
 * summation order, which each reproduces exactly.
 * RING: each chunk c of q = ceil(n/p) elements is folded in the ring
 *   order x_{c+1}, x_{c+2}, ..., x_c (indices mod p) with the partial kept
 *   on chip across the p-1 combine steps, then stored to all p outputs in
 *   the same pass (reduce-scatter and all-gather fused).  Bit-exact with
 *   the ring all-reduce of [A] 2.2 read with chunk c ending on rank c.
 * ONEPASS (= RECURSIVE_DOUBLING): all p inputs summed as the balanced
 *   tree that recursive doubling builds when rank r exchanges with
 *   r XOR 2^k at step k = 0, 1, ... ([A] 2.3): (x0+x1), (x2+x3), ... first.
 *   Every rank gets the same bits.  p in {2,4,8,16}.
 * RING_LITERAL: the 2(p-1) neighbour steps of [A] 2.2 run one step per
 *   kernel launch through HBM, partials stored in the receive buffers.
 *   Bit-exact with RING.  fp32 and int32 only.
 * HALVING_DOUBLING: the order of [A] 2.3's halving-doubling, read as a
 *   recursive-halving reduce-scatter pairing ranks at distance p/2, p/4,
 *   ..., 1 followed by a recursive-doubling all-gather:
 *   (x0 + x_{p/2}), (x1 + x_{p/2+1}), ... first.  p in {2,4,8,16}.
 * TREE: the tree all-reduce ([B] Tree AllReduce: reduce up a binary tree
 *   to the root, then broadcast down), the tree in heap order (rank v's
 *   children 2v+1 and 2v+2): each node adds its own value, then its left
 *   subtree, then its right.  2 <= p <= 16.
 * DOUBLE_BINARY_TREE: [A] 2.4's two complementary trees, tree A as TREE
 *   and tree B its mirror (node v on rank p-1-v); chunks c < p/2 (rounded
 *   down) of q = ceil(n/p) elements are reduced on tree A, the others on
 *   tree B.  2 <= p <= 16.
 * A schedule outside these rank counts returns COLL_ERR_UNSUPPORTED.
 * Integer sums and min/max give the same bits under every schedule. */
typedef enum {
  COLL_ALGO_RING = 0,
  COLL_ALGO_ONEPASS = 1,
  COLL_ALGO_RECURSIVE_DOUBLING = 1,
  COLL_ALGO_RING_LITERAL = 2,
  COLL_ALGO_HALVING_DOUBLING = 3,
  COLL_ALGO_TREE = 4,
  COLL_ALGO_DOUBLE_BINARY_TREE = 5
} coll_algo_t;

#define COLL_MAX_RANKS 64

/* AllReduce ([A] 1.4, [B] AllReduce): recv[r][i] = (+)_{r'} send[r'][i]
 * for every rank r and i < n.  Same as coll_allreduce_algo with
 * COLL_ALGO_RING.  send[r], recv[r]: n elements each.
 * In place: recv[r] == send[r]. */
coll_status_t coll_allreduce(const void* const* send, void* const* recv, int p, size_t n,
                             coll_dtype_t dtype, coll_op_t op, void* stream);

/* AllReduce with an explicit schedule (see coll_algo_t). */
coll_status_t coll_allreduce_algo(const void* const* send, void* const* recv, int p, size_t n,
                                  coll_dtype_t dtype, coll_op_t op, coll_algo_t algo,
                                  void* stream);

/* Pre-multiplied AllReduce ([B] numerics: NCCL's PreMulSum, the one
 * constrained custom reduction): recv[r][i] = sum_k scale[k] * send[k][i],
 * each operand multiplied by its rank's scale in fp32 and rounded on its
 * own, then summed in the order of `algo` (any schedule but RING_LITERAL).  scale: HOST array of p floats.  fp32 and bf16 only
 * (COLL_ERR_UNSUPPORTED for int32 and RING_LITERAL).  In place as
 * coll_allreduce.  scale = 1/p for every rank is the average of DDP. */
coll_status_t coll_allreduce_premul(const void* const* send, void* const* recv, int p, size_t n,
                                    coll_dtype_t dtype, const float* scale, coll_algo_t algo,
                                    void* stream);

/* Reduce ([A] 1.3 with its worked example): recv_root[i] = (+)_r send[r][i];
 * only the root's buffer is written.  Same summation order as
 * coll_allreduce, so Reduce then Broadcast equals AllReduce bit for bit.
 * root in [0, p) is a rank index.  In place: recv_root == send[root]. */
coll_status_t coll_reduce(const void* const* send, void* recv_root, int p, size_t n,
                          coll_dtype_t dtype, coll_op_t op, int root, void* stream);

/* Broadcast ([A] 1.1): recv[r][i] = send_root[i] for every r, i < n.
 * root in [0, p).  In place: recv[root] == send_root. */
coll_status_t coll_broadcast(const void* send_root, void* const* recv, int p, size_t n,
                             coll_dtype_t dtype, int root, void* stream);

/* ReduceScatter ([A] 1.5): send[r] holds p*n elements, recv[r] holds n;
 * recv[r][j] = (+)_k send[k][r*n + j], block r folded in the ring order
 * x_{r+1}, ..., x_r.  In place: recv[r] == send[r] + r*n elements. */
coll_status_t coll_reduce_scatter(const void* const* send, void* const* recv, int p, size_t n,
                                  coll_dtype_t dtype, coll_op_t op, void* stream);

/* Pre-multiplied ReduceScatter: as coll_reduce_scatter with op sum, each
 * rank's operand first multiplied by scale[rank] (HOST array of p floats),
 * products rounded to fp32 on their own.  fp32 and bf16 only. */
coll_status_t coll_reduce_scatter_premul(const void* const* send, void* const* recv, int p, size_t n,
                                         coll_dtype_t dtype, const float* scale, void* stream);

/* AllGather ([A] 1.2): send[s] holds n elements, recv[r] holds p*n;
 * recv[r][s*n + j] = send[s][j] (rank-order concatenation).
 * In place: send[r] == recv[r] + r*n elements. */
coll_status_t coll_allgather(const void* const* send, void* const* recv, int p, size_t n,
                             coll_dtype_t dtype, void* stream);

/* All-to-All, equal split ([A] 1.6): send[i] and recv[j] hold p blocks of
 * n_block elements; recv[j][i*n_block + k] = send[i][j*n_block + k], the
 * transpose of the p x p block matrix.  No in-place form. */
coll_status_t coll_alltoall(const void* const* send, void* const* recv, int p, size_t n_block,
                            coll_dtype_t dtype, void* stream);

/* How the All-to-All block transpose moves its bytes.  Both give the same
 * result (a bit copy).
 * DIRECT: 16-byte vectors go from the source block to the destination
 *   block through registers (what coll_alltoall does).
 * LDS_STAGED: every vector is staged in LDS on the way: gfx950 loads
 *   global memory straight into LDS, each wave alternating two private
 *   stages of 8 KiB, one filling while the other is written out.  It needs
 *   every block to share one 16-byte misalignment: the send and the recv
 *   buffers share a misalignment and n_block * element size is a multiple
 *   of 16.  Other layouts run the DIRECT kernel. */
typedef enum { COLL_A2A_DIRECT = 0, COLL_A2A_LDS_STAGED = 1 } coll_a2a_algo_t;

/* All-to-All ([A] 1.6) with an explicit data path (see coll_a2a_algo_t);
 * arguments, layout and errors as coll_alltoall, plus
 * COLL_ERR_INVALID_ARG for an unknown algo. */
coll_status_t coll_alltoall_algo(const void* const* send, void* const* recv, int p, size_t n_block,
                                 coll_dtype_t dtype, coll_a2a_algo_t algo, void* stream);

/* Gather ([C] section 4.3; [A] note after 1.6): AllGather whose result
 * only the root keeps.  send[s] holds n elements, recv_root holds p*n;
 * recv_root[s*n + j] = send[s][j] (rank-order concatenation).  root in
 * [0, p).  In place: send[root] == recv_root + root*n elements. */
coll_status_t coll_gather(const void* const* send, void* recv_root, int p, size_t n,
                          coll_dtype_t dtype, int root, void* stream);

/* Scatter ([C] section 3.3; [A] note after 1.6): the root's p*n elements
 * cut into p blocks of n, block r to rank r: recv[r][j] =
 * send_root[r*n + j].  root in [0, p).  In place: recv[root] ==
 * send_root + root*n elements. */
coll_status_t coll_scatter(const void* send_root, void* const* recv, int p, size_t n,
                           coll_dtype_t dtype, int root, void* stream);

/* Variable-split All-to-All ([B] Ragged All-to-All).
 * counts_dev: DEVICE array of p*p int64, row-major, counts[i*p + j] =
 *   elements source i sends to destination j (as produced on the device by
 *   a router).  Send offsets are the exclusive prefix sums along row i;
 *   recv[j] receives the blocks of sources 0..p-1 packed in source order.
 * send_cap, recv_cap: HOST arrays of p int64, the capacity in elements of
 *   send[i] and recv[j].  The kernel checks on the device that every count
 *   is >= 0, that row sums fit send_cap and column sums fit recv_cap; if
 *   not it writes no payload at all.
 * status_dev: optional DEVICE int32 (may be NULL).  The kernel stores 0 on
 *   success or COLL_ERR_INVALID_ARG when the counts were rejected.
 * No in-place form; the counts array may not overlap any recv buffer. */
coll_status_t coll_alltoallv(const void* const* send, void* const* recv, int p,
                             const int64_t* counts_dev, const int64_t* send_cap,
                             const int64_t* recv_cap, int32_t* status_dev,
                             coll_dtype_t dtype, void* stream);

/* The reverse of coll_alltoallv ([A] 1.7 duality table: All-to-All is
 * its own dual with the splits swapped; [B] Ragged All-to-All: "reverse
 * variable-split All-to-All").  counts_dev is the FORWARD matrix: the
 * elements going from rank i to rank j now are counts_dev[j*p + i].
 * Otherwise as coll_alltoallv (capacities, device-side checks, status). */
coll_status_t coll_alltoallv_transposed(const void* const* send, void* const* recv, int p,
                                        const int64_t* counts_dev, const int64_t* send_cap,
                                        const int64_t* recv_cap, int32_t* status_dev,
                                        coll_dtype_t dtype, void* stream);

/* MoE dispatch pack ([B] Ragged All-to-All flow "count assignments per
 * destination -> prefix-sum offsets -> pack/permute payload"; [B] Expert
 * Parallel: the unit is the assignment, not the token).
 * Per rank i: tokens[i] holds T rows of `hidden` elements; dest[i] (device
 * int32, T*k) is the destination rank of assignment a = t*k + s.
 * Assignments are ordered by destination rank, stable in a.  Outputs:
 *   pos[i][a]      packed row of assignment a (device int32, T*k);
 *   packed[i]      T*k rows: row pos[i][a] = token a / k;
 *   counts_dev     [p][p] int64, counts[i][j] = hidden * (assignments of
 *                  rank i to rank j): the forward matrix for
 *                  coll_alltoallv, then coll_alltoallv_transposed;
 *   status_dev     optional device int32[p]: 0, or 1 if rank i had a
 *                  destination outside [0, p); such a rank gets counts 0,
 *                  every pos -1 and no payload.
 * k in [1, 8]; T = 0 writes zero counts.  No output may overlap another
 * buffer. */
coll_status_t coll_moe_pack(const void* const* tokens, const int32_t* const* dest, void* const* packed,
                            int32_t* const* pos, int64_t* counts_dev, int32_t* status_dev, int p,
                            size_t tokens_per_rank, int k, size_t hidden, coll_dtype_t dtype,
                            void* stream);

/* MoE weighted combine ([B] Expert Parallel: "weighted combine +
 * residual", after the reverse exchange and the unpermute).  back[i] holds
 * rank i's T*k returned rows in packed order; for every token t
 *   out[i][t] = r + w[i][t*k] * back[i][pos[i][t*k]] + ... + w[i][t*k+k-1] * ...
 * with r = residual[i][t] (residual may be NULL: r = +0), accumulated in
 * fp32 in slot order, every product and sum rounded to fp32 on its own (no
 * fused multiply-add), bf16 narrowed once.  weights: device fp32 (T*k).
 * Slots whose pos is outside [0, T*k) are skipped.  fp32 and bf16 only
 * (COLL_ERR_UNSUPPORTED for int32).  In place: out[i] == residual[i]. */
coll_status_t coll_moe_combine(const void* const* back, const int32_t* const* pos,
                               const float* const* weights, const void* const* residual,
                               void* const* out, int p, size_t tokens_per_rank, int k, size_t hidden,
                               coll_dtype_t dtype, void* stream);

/* FP8 e4m3 dispatch ([A] 4.3 quantized communication: the dispatch
 * payload travels as FP8 e4m3, the combine stays bf16, halving the
 * dispatch bytes).  Format: OCP E4M3 (sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, subnormals m * 2^-9, no infinities, S.1111.111 NaN,
 * largest finite 448).  Each token row of `hidden` bf16 values is cut into
 * groups of `group` consecutive elements; per group, in fp32 with every
 * operation rounded to nearest even:
 *   amax  = max(max |x|, 2^-110),  inv = 448 / amax,  scale = amax / 448,
 *   code  = e4m3(x * inv), round to nearest even, saturating at +-448.
 * Packed row (coll_moe_fp8_row_bytes(hidden, group) bytes, a multiple of
 * 16): the hidden codes, then the hidden/group fp32 scales, then zero
 * bytes.  Shapes: group divides hidden; group is a power of two in
 * [16, 1024] or a multiple of 1024; hidden < 2^31, and hidden <= 16384
 * when group > 1024 (else COLL_ERR_UNSUPPORTED).  Non-finite inputs give
 * unspecified codes. */

/* Bytes of one packed FP8 row, or 0 if (hidden, group) is not accepted. */
size_t coll_moe_fp8_row_bytes(size_t hidden, size_t group);

/* Quantizing dispatch pack: coll_moe_pack for bf16 tokens, writing FP8
 * rows.  tokens[i]: T rows of `hidden` bf16; dest, pos, status_dev as
 * coll_moe_pack; packed[i]: T*k rows of row_bytes bytes, row pos[i][a]
 * the encoded token a / k; counts_dev [p][p] int64 in BYTES (rows *
 * row_bytes), the forward matrix for coll_alltoallv with COLL_U8;
 * counts_hidden_dev (optional, may be NULL) the same matrix in rows *
 * hidden, the forward matrix of the bf16 reverse exchange
 * (coll_alltoallv_transposed of the experts' bf16 rows).  tokens and
 * packed must be 16-byte aligned.  No output may overlap another buffer. */
coll_status_t coll_moe_pack_fp8(const void* const* tokens, const int32_t* const* dest,
                                void* const* packed, int32_t* const* pos, int64_t* counts_dev,
                                int64_t* counts_hidden_dev, int32_t* status_dev, int p,
                                size_t tokens_per_rank, int k, size_t hidden, size_t group,
                                void* stream);

/* Dequantization of received FP8 rows for a bf16 consumer:
 * y = bf16(decode(code) * scale), the product rounded to fp32 first.
 * Rank j received sum_i counts_dev[i*p + j] bytes (the forward matrix of
 * coll_moe_pack_fp8, after coll_alltoallv): recv[j] holds those rows in
 * arrival order, out[j] gets the same number of bf16 rows of `hidden`.
 * rows_cap: host int64[p], rows that recv[j] and out[j] hold.  Checked on
 * the device: every count a non-negative multiple of row_bytes and each
 * rank's total within rows_cap; otherwise nothing is written and
 * *status_dev (optional device int32) is 1, else 0.  recv and out must be
 * 16-byte aligned and may not overlap. */
coll_status_t coll_moe_dequant_fp8(const void* const* recv, void* const* out, int p,
                                   const int64_t* counts_dev, const int64_t* rows_cap,
                                   int32_t* status_dev, size_t hidden, size_t group, void* stream);

/* Direct MoE dispatch ([B] Ragged All-to-All flow and Expert Parallel;
 * [A] 3.9: kernels that load and store peers' buffers directly): the pack
 * and the dispatch exchange in one pass, with no staging buffer.  Every
 * assignment's token row is written straight into its destination's
 * receive buffer, in the layout coll_moe_pack followed by coll_alltoallv
 * produces (source ranks in order, each source's rows in assignment
 * order).
 *   recv[j]      the rows rank j receives; recv_cap: HOST int64[p], rows
 *                each recv[j] holds (at most 2^31 - 1);
 *   loc[i][a]    device int64 (T*k): (dest << 32) | row inside recv[dest],
 *                or -1 when assignment a is not delivered; the handle
 *                coll_moe_combine_direct reads;
 *   counts_dev   [p][p] int64 = hidden * rows, as coll_moe_pack;
 *   status_dev   optional device int32[p + 1]: entries 0..p-1 as
 *                coll_moe_pack (1: the rank had a destination outside
 *                [0, p) and its locations are -1); entry p is 1 when some
 *                rank would receive more rows than its capacity, and then
 *                no payload is written and every location is -1.
 * Any dtype (COLL_U8 included); tokens and recv aligned to the element
 * size; k in [1, 8].  No output may overlap another buffer. */
coll_status_t coll_moe_dispatch(const void* const* tokens, const int32_t* const* dest, void* const* recv,
                                int64_t* const* loc, int64_t* counts_dev, int32_t* status_dev, int p,
                                size_t tokens_per_rank, int k, size_t hidden, const int64_t* recv_cap,
                                coll_dtype_t dtype, void* stream);

/* Direct FP8 dispatch: coll_moe_dispatch with the encoded rows of
 * coll_moe_pack_fp8 (bf16 tokens; rows of coll_moe_fp8_row_bytes bytes,
 * recv_cap counted in those rows); counts_dev in bytes, counts_hidden_dev
 * (optional) in rows * hidden.  tokens and recv 16-byte aligned. */
coll_status_t coll_moe_dispatch_fp8(const void* const* tokens, const int32_t* const* dest, void* const* recv,
                                    int64_t* const* loc, int64_t* counts_dev, int64_t* counts_hidden_dev,
                                    int32_t* status_dev, int p, size_t tokens_per_rank, int k, size_t hidden,
                                    size_t group, const int64_t* recv_cap, void* stream);

/* Combine reading the experts' outputs where they lie, in place of
 * coll_alltoallv_transposed followed by coll_moe_combine: y[j] holds
 * y_rows[j] (HOST int64, at most 2^31 - 1) output rows of `hidden`
 * elements in rank j's receive order; loc comes from coll_moe_dispatch or
 * coll_moe_dispatch_fp8.  For every token t of rank i
 *   out[i][t] = r + sum_s w[i][t*k+s] * y[loc >> 32][loc & 0xffffffff]
 * with loc = loc[i][t*k+s] and the arithmetic of coll_moe_combine (fp32,
 * slot order, each product and sum rounded, bf16 narrowed once).
 * Locations that are -1, name a rank >= p or a row >= y_rows are skipped.
 * fp32 and bf16 (COLL_ERR_UNSUPPORTED for int32).  In place: out[i] ==
 * residual[i]. */
coll_status_t coll_moe_combine_direct(const void* const* y, const int64_t* const* loc,
                                      const float* const* weights, const void* const* residual,
                                      void* const* out, int p, size_t tokens_per_rank, int k, size_t hidden,
                                      const int64_t* y_rows, coll_dtype_t dtype, void* stream);

/* One AllReduce of a batch (host-side view). */
typedef struct {
  const void* const* send;  /* host array of p device pointers */
  void* const* recv;        /* host array of p device pointers */
  size_t n;                 /* elements per rank */
  coll_dtype_t dtype;
  coll_op_t op;
} coll_call_t;

/* Flags for coll_allreduce_batch. */
#define COLL_BATCH_CHECK_ALIAS 1u  /* also reject overlaps between calls (O(m log m) host work) */

/* Batched AllReduce ([B] group calls; [A] 4.2 bucketing/fusion): ncalls
 * independent AllReduces over the same p, enqueued as one kernel launch so
 * that the fixed per-call cost is paid once.  Each call has the semantics
 * and summation order of coll_allreduce; calls may mix dtypes and ops.
 * Within a call the coll_allreduce aliasing rules always apply; overlaps
 * between calls are checked only with COLL_BATCH_CHECK_ALIAS (otherwise
 * overlapping calls race).  The library copies the descriptors into one
 * of two device buffers it owns, used in turn (grown on demand, released
 * by coll_finalize); a call waits on the host only for the batch kernel
 * two calls earlier, the last one to use the same buffer, so the host
 * prepares a batch while the one before it runs. */
coll_status_t coll_allreduce_batch(const coll_call_t* calls, int ncalls, int p,
                                   unsigned flags, void* stream);

/* Batched AllReduce that allocates nothing, for callers that cannot call
 * hipMalloc (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, validation, semantics, order
 * and kernels as coll_allreduce_batch, but the descriptor table (call
 * records and pointer lists) goes to a static device array of
 * COLL_BATCH_NOALLOC_MAX_BYTES that every GPU the library runs on holds
 * until the process ends; nothing is allocated and nothing waits on the
 * host for earlier batches.  The table takes
 *   ((32 * (ncalls + 1) + 255) / 256) * 256 + 256 + 16 * p * ncalls   bytes
 * (10,000 calls at p = 16 fit); a larger batch returns
 * COLL_ERR_INVALID_ARG before anything is enqueued.  The table is copied
 * with hipMemcpyAsync on `stream` from a static host buffer (pageable
 * memory: HIP has read it when the copy call returns; calls from several
 * host threads take turns).  All calls on one GPU share that GPU's table,
 * which keeps the last call's contents: calls on one stream are ordered,
 * while calls that overlap on different streams of one GPU race (a later
 * upload can overwrite descriptors an earlier kernel still reads). */
#define COLL_BATCH_NOALLOC_MAX_BYTES (4u << 20)
coll_status_t coll_allreduce_batch_noalloc(const coll_call_t* calls, int ncalls, int p, unsigned flags,
                                           void* stream);

/* Direction-mix bandwidth probe: a measurement helper, not a collective.
 * [A] 4.1 models a collective's time by the bandwidth of each resource it
 * uses, and [A] 2.5 compares bus bandwidth with what the hardware
 * sustains; on one device the resource is HBM, and what it sustains
 * depends on how many read and write streams are in flight.  This call
 * streams `nsrc` sources and `ndst` destinations of `bytes` bytes each
 * through the collectives' 16-byte vector tiles of `unroll` vectors per
 * lane (1, 2, 4 or 8, with nsrc * unroll <= 32; every load of a tile is
 * issued before its first store), with the reductions' launch bounds and
 * default grid (coll_set_grid_limit applies):
 * every destination receives the XOR of the sources' 32-bit words (a
 * fixed pattern when nsrc == 0).  With ndst == 0 the loads are folded into
 * one value per lane that is written to `sink` (16 device bytes, 16-byte
 * aligned) only if it equals an internal pattern, so the reads stay.
 * flags: COLL_PROBE_NT_LOADS / COLL_PROBE_NT_STORES select non-temporal
 * loads / stores (else cached); COLL_PROBE_DEVICE_STORES makes the stores
 * of device scope, written through the L2 as ReduceScatter and Reduce
 * store (with COLL_PROBE_NT_STORES: non-temporal stores of device scope,
 * as AllGather and Broadcast at p >= 2 store);
 * COLL_PROBE_CLAIM deals out about a quarter
 * of the tiles in turn and lets workgroups claim the rest one at a time
 * from eight pooled counters, as the large copies and reductions balance
 * their work (with at least 8 whole tiles per workgroup and 64 workgroups;
 * else every tile is dealt out).  Supported (nsrc, ndst): (1|4|8|16, 0),
 * (0, 1|4|8|16), (1|2|3|4|5|6|7|8|12|16, 1), (1, 2|4|8|16) and (k, k) for
 * k in 3, 4, 5, 6, 7, 8, 12, 16; other pairs and tile sizes return
 * COLL_ERR_UNSUPPORTED.  Every pointer
 * 16-byte aligned and bytes a multiple of 16 (else COLL_ERR_INVALID_ARG);
 * destinations may not overlap each other or a source (COLL_ERR_ALIAS). */
#define COLL_PROBE_NT_LOADS 1u
#define COLL_PROBE_NT_STORES 2u
#define COLL_PROBE_CLAIM 4u
#define COLL_PROBE_DEVICE_STORES 8u
coll_status_t coll_stream_probe(const void* const* src, int nsrc, void* const* dst, int ndst, size_t bytes,
                                int unroll, unsigned flags, void* sink, void* stream);

/* Human-readable name of a status code (static storage). */
const char* coll_status_string(coll_status_t status);

/* The last hipError_t recorded by a call on this host thread that
 * returned COLL_ERR_HIP (0 if none). */
int coll_last_hip_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int coll_version(void);

/* Occupancy target used to size grids: workgroups (256 threads) per
 * compute unit, for every kernel; 0 restores each kernel family's
 * measured default (1 for reductions, 2 for copies and the direct FP8
 * dispatch, 8 for the MoE row kernels, 16 for the FP8 pack and dequant).
 * Negative values count as 0; values above 64 are clamped to 64.
 * Applies to later calls from every thread; results do not depend on it. */
void coll_set_grid_limit(int workgroups_per_cu);

/* Release library-owned device and pinned host memory (batch descriptors).
 * Synchronises on the work that used them. */
void coll_finalize(void);

#ifdef __cplusplus
}
#endif

#endif /* COLL_H_ */
