/*
 * sgemv.h - C ABI of the MI355X (gfx950) SparseGemv library.
 *
 * What it computes: y = W' x, where W' is a weight matrix pruned to a
 * semi-structured N:M pattern along the input dimension (2:4 for important
 * layers, 1:4 for the others), quantised to INT4 with asymmetric group-wise
 * scales whose group size is chosen per output channel, and stored in an
 * index-compressed "2bit-CSR" format; x is FP16 (one vector or a small beam
 * batch) and accumulation is FP32. Source: the page "Efficient large-model
 * ad applications through model compression and parallel verification"
 * (English gloss of its Chinese title; a Chinese translation of arXiv
 * 2605.11582), cited as P1 below: §1 ("our core idea"
 * and the contribution list), §3.2 "Model compression" (adaptive group
 * quantization, sparsification, eqs. (1)-(3)) and §3.3 "Revised kernel".
 *
 * Conventions
 *  - W is N x K, row-major, row n = output channel, column k = input
 *    channel; y[b][n] = sum_k W'[n][k] * x[b][k].
 *  - FP16 values travel as their uint16 bit patterns.
 *  - Every function returns an int status: SGEMV_OK (0) or a negative error
 *    code. Nothing aborts, throws or prints. All checks except SGEMV_EHIP
 *    happen on the host before any HIP call.
 *  - The library allocates no memory visible to the caller and is
 *    re-entrant. Its only state is a record of the kernels whose LDS limit
 *    it has raised on a device (HIP keeps that attribute per kernel and
 *    device, so it is set once), guarded by a mutex. Host arrays are owned and sized by the caller;
 *    device buffers are owned by the caller (e.g. torch tensors).
 */
#ifndef SGEMV_H
#define SGEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SGEMV_OK = 0,
  SGEMV_EINVAL = -1, /* bad shape, N:M choice, group size, batch, NULL pointer, non-finite weight */
  SGEMV_ESIZE = -2,  /* inconsistent descriptor, or a size beyond what the kernels support */
  SGEMV_EALIGN = -3, /* a device pointer is not aligned as required */
  SGEMV_EHIP = -4    /* the HIP runtime reported an error at launch */
};

/* Plain-data description of one packed layer. Filled by sgemv_describe and
 * passed back by pointer; the caller may copy it freely. */
typedef struct sgemv_desc {
  int32_t N, K;          /* output rows, input columns (K % 256 == 0)                  */
  int32_t nk;            /* kept per group of 4 along K: 2 (2:4), 1 (1:4), 4 (dense)   */
  int32_t n_blocks;      /* row blocks of 16 rows (rows sorted by group size)          */
  int32_t chunks;        /* column chunks of 256 dense columns per row: K / 256        */
  int32_t g_min, g_max;  /* smallest and largest group size present                    */
  int32_t class_rows[4]; /* rows with group size 32, 64, 128, 256 (sorted in that order) */
  int32_t value_format;  /* 0: INT4 codes with group scale/zero; 1: FP16 values       */
  int64_t kept;          /* N*K*nk/4 kept elements                                     */
  int64_t vals_bytes;    /* canonical value array: kept/2 bytes (INT4), kept*2 (FP16)  */
  int64_t offs_bytes;    /* canonical offset array: kept/4 bytes (2 bits each); 0 dense */
  int64_t n_groups;      /* sum_n K/g_n: one FP16 scale and one FP16 zero each         */
  int64_t off_codes;     /* byte offsets of the blob sections (256-byte aligned)       */
  int64_t off_offs;
  int64_t off_perm;
  int64_t off_sz;
  int64_t blob_bytes;    /* total size of the kernel-layout blob                       */
} sgemv_desc;

/* sgemv_describe - validate a layer shape and fill its descriptor.
 *   N, K         : rows and columns; N >= 1, K >= 256, K % 256 == 0, K <= 32768,
 *                  and the blob must stay below 2^31 bytes.
 *   nk           : 2 for 2:4 or 1 for 1:4 (P1 §3.2 "Sparsification"); 4 for
 *                  the dense INT4 ablation (every element kept, no offsets:
 *                  the plain weight-only GEMV that SparseGemv extends, P1 §1
 *                  contributions, second item), which sgemv_pack,
 *                  sgemv_layout and sgemv_run accept as well.
 *   group_size   : host int32[N], group size of each row in dense columns; each
 *                  in {32, 64, 128, 256} (P1 §3.2 "Adaptive group quantization":
 *                  finer groups for sensitive channels).
 *   out          : filled on success.
 * Errors: EINVAL for bad arguments, ESIZE beyond the supported sizes. */
int sgemv_describe(int32_t N, int32_t K, int32_t nk, const int32_t* group_size,
                   sgemv_desc* out);

/* sgemv_describe_fp16 - descriptor of the FP16-valued form: the same N:M
 * selection and 2-bit offsets, each kept value stored as FP16 (no groups, no
 * scale or zero): the semi-structured layer-wise FP16 mixed sparsity of P1 §1
 * ("our core idea") before INT4 compression.
 *   N, K, nk : as sgemv_describe (nk 1 or 2).
 * The descriptor has value_format 1, n_groups 0, no class rows, and its blob
 * holds values [blocks][chunks][64 lanes][32*nk bytes] (each lane's 16*nk
 * kept values in element order), offsets as the INT4 form, and perm (the
 * identity: there are no group sizes to sort by).
 * Errors: EINVAL, ESIZE as sgemv_describe. */
int sgemv_describe_fp16(int32_t N, int32_t K, int32_t nk, sgemv_desc* out);

/* sgemv_select_groups - adaptive group size per output channel (P1 §3.2
 * "Adaptive group quantization"; sensitivity from the first term of eq. (3)).
 *   w            : host FP16 bits [N][K], dense weights (pruned inside, as sgemv_pack).
 *   xcal, T      : host FP16 bits [T][K], calibration activations, T >= 1.
 *   frac_fine    : fraction of rows given the fine size, in [0, 1], taken to 6
 *                  decimals; the count is ceil(N * frac_fine).
 *   g_fine, g_coarse : group sizes (each valid for sgemv_describe).
 *   group_size_out   : host int32[N].
 * With c_k = sqrt(sum_t xcal[t][k]^2) and S_n = sum_k |Wp[n][k]| * c_k (FP64,
 * sequential sums in index order, Wp = W after N:M pruning), the rows with the
 * largest S_n (ties: lower n) get g_fine and all others g_coarse.
 * Errors: EINVAL (shape, NULL, non-finite weight or activation, bad sizes). */
int sgemv_select_groups(const uint16_t* w, int32_t N, int32_t K, int32_t nk,
                        const uint16_t* xcal, int32_t T, double frac_fine,
                        int32_t g_fine, int32_t g_coarse, int32_t* group_size_out);

/* sgemv_prune - N:M pruning by the activation-aware importance of P1 §3.2
 * (eq. (3), first term): score(n, k) = |w[n][k]| * c_k with
 * c_k = sqrt(sum_t xcal[t][k]^2) (FP64, sequential over t). In every group of
 * 4 consecutive columns of a row the nk largest scores are kept (ties: lower
 * column); the gradient term of eq. (3) is not used (it needs a loss).
 *   w      : host FP16 bits [N][K], dense weights.
 *   xcal, T: host FP16 bits [T][K] calibration activations, T >= 1; NULL for
 *            unit column scales (score |w|, the selection sgemv_pack makes).
 *   w_out  : host FP16 bits [N][K]: the kept values, bits unchanged, and +0
 *            at pruned positions (may not alias w).
 * Passing w_out to sgemv_select_groups / sgemv_pack reproduces the same
 * pruned matrix: their |w| selection keeps every non-zero of a group that
 * has at most nk non-zeros, and kept zeros dequantise to zero wherever they
 * sit. Errors: EINVAL (shape, NULL, T < 1 with xcal, non-finite values). */
int sgemv_prune(const uint16_t* w, int32_t N, int32_t K, int32_t nk,
                const uint16_t* xcal, int32_t T, uint16_t* w_out);

/* sgemv_pack - dense FP16 W -> N:M prune -> asymmetric INT4 group quantisation
 * -> canonical 2bit-CSR arrays (P1 §1 contributions, first item; §3.2).
 * Pruning keeps, in every group of 4 consecutive columns of a row, the nk
 * elements of largest |w| (ties: lower column), offsets ascending. Each
 * (row, group) is quantised over its kept values: lo = min(0, min v),
 * hi = max(0, max v); scale = fp16((hi - lo) / 15) (1 if hi == lo, at least
 * 2^-24); zero = clamp(rint(-lo/scale), 0, 15); code = clamp(rint(v/scale) +
 * zero, 0, 15); FP64 arithmetic, round half to even.
 * Output arrays (host, caller-sized from the descriptor):
 *   vals  [N][K*nk/8]  element j of a row in byte j/2, low nibble when j is even;
 *   offs  [N][K*nk/16] in-group offset of element j in byte j/4, bits 2(j%4)..+1
 *                      (none, and offs may be NULL, for the dense nk = 4);
 *   scale, zero [n_groups] FP16 bits, row-major over (row, group);
 *   gptr  [N+1] first group of each row; rowptr [N+1] = n*K*nk/4.
 * Errors: EINVAL (shape, group sizes, NULL, non-finite weight). */
int sgemv_pack(const uint16_t* w, int32_t N, int32_t K, int32_t nk,
               const int32_t* group_size, uint8_t* vals, uint8_t* offs,
               uint16_t* scale, uint16_t* zero, int32_t* gptr, int32_t* rowptr);

/* sgemv_pack_fp16 - dense FP16 W -> N:M prune (as sgemv_pack) -> FP16-valued
 * 2bit-CSR: vals16 [N][K*nk/4] FP16 bits of kept element j (ascending column),
 * offs [N][K*nk/16] as sgemv_pack, rowptr [N+1] = n*K*nk/4 (host arrays).
 * Errors: EINVAL (shape, nk not 1 or 2, NULL, non-finite weight). */
int sgemv_pack_fp16(const uint16_t* w, int32_t N, int32_t K, int32_t nk,
                    uint16_t* vals16, uint8_t* offs, int32_t* rowptr);

/* sgemv_layout_fp16 - FP16-valued canonical arrays -> kernel-layout blob
 * (host buffer of d->blob_bytes, fully written); d from sgemv_describe_fp16.
 * Errors: EINVAL (NULL, a descriptor of the other format), ESIZE. */
int sgemv_layout_fp16(const sgemv_desc* d, const uint16_t* vals16, const uint8_t* offs, void* blob);

/* sgemv_layout - canonical arrays -> kernel-layout blob (host). The blob holds
 * the same bits reordered for the matrix-core kernel (no duplication; zero
 * padding only for the rows of a last, partial row block):
 *  - rows sorted by group size (ascending, stable); row block b = sorted rows
 *    16b..16b+15; a piece = one row's kept elements in 64 dense columns;
 *  - 2:4: codes [blocks][chunks][64 lanes][16 bytes] and offsets
 *    [blocks][chunks][64 lanes][8 bytes]; 1:4: one section
 *    [blocks][chunks][64 lanes][12 bytes], a lane's 2 code dwords then its
 *    offset dword, and an empty offset section; lane r + 16q of record
 *    (b, c) holds the piece of sorted row 16b + r in columns 256c + 64q ..
 *    +63, with a fixed nibble order inside each code dword and, at 1:4, a
 *    fixed 2-bit order inside the offset dword;
 *  - perm int32[16*blocks]: original row of each sorted row, -1 for padding;
 *  - scale|zero<<16 words in records (b, c), each listing the rows of block b
 *    in order with their 256/g words of chunk c.
 * The exact bit positions are listed with the layout builder (host_layout.cpp)
 * and the oracle's layout module. Group sizes are taken from gptr.
 *   d        : descriptor from sgemv_describe for the same group sizes.
 *   blob     : host buffer of d->blob_bytes bytes, fully written.
 * The kernel holds each weight as the FP16 value (code - zero) * scale, rounded
 * once; a layer where that value rounds beyond the FP16 range (|value| >=
 * 65520, possible only for groups reaching within 2^-11 of the FP16 maximum)
 * is rejected with EINVAL.
 * Errors: EINVAL (NULL, gptr inconsistent with d, FP16 range), ESIZE. */
int sgemv_layout(const sgemv_desc* d, const uint8_t* vals, const uint8_t* offs,
                 const uint16_t* scale, const uint16_t* zero, const int32_t* gptr,
                 void* blob);

/* sgemv_run - y = W' x on the GPU (P1 §3.3 "Revised kernel": INT4 weight-only
 * GEMV with mixed N:M sparsity).
 *   d        : descriptor of the packed layer.
 *   blob_dev : device copy of the blob, 256-byte aligned, d->blob_bytes bytes.
 *   x_dev    : device FP16 [B][K] row-major, 16-byte aligned.
 *   y_dev    : device FP16 [B][N] row-major, 2-byte aligned; fully overwritten.
 *   B        : batch (beam width), 1..16.
 *   hip_stream : hipStream_t to enqueue on (NULL = default stream).
 * Numerics: each weight enters as FP16 (code - zero) * scale (one rounding,
 * relative error <= 2^-11), products and sums in FP32, y rounded to FP16;
 * |y - W'x| <= (2^-11 + n 2^-24) sum_k |W'[n][k] x[k]| + 2^-11 |y| for n
 * kept elements per row (FP16-valued layers: the weights enter exactly, and
 * the first term drops to n 2^-24). Both value formats are accepted. Non-finite x gives non-finite rows, as the dense
 * product does.
 * Enqueues one kernel and returns without synchronising. x and y must not
 * overlap the blob or each other. Deterministic: the same inputs give the
 * same bits on every call. Errors: EINVAL, ESIZE, EALIGN (host checks), EHIP. */
int sgemv_run(const sgemv_desc* d, const void* blob_dev, const void* x_dev,
              void* y_dev, int32_t B, void* hip_stream);

/* What sgemv_run enqueues for a layer and a batch (filled by sgemv_plan). */
typedef struct sgemv_plan_t {
  int64_t grid;            /* workgroups launched: ceil(row blocks / row_blocks)      */
  int64_t lds_bytes;       /* dynamic LDS per workgroup (x slices and wave partials)  */
  int32_t block;           /* lanes per workgroup: 64 * waves                         */
  int32_t waves;           /* waves per workgroup; wave w owns a contiguous range of   */
                           /* column chunks: chunks_per_wave of them if              */
                           /* w < full_waves, one less after (fewer at the row end), */
                           /* starting at w * chunks_per_wave - max(0, w - full_waves) */
  int32_t chunks_per_wave;
  int32_t phase_chunks;    /* chunks whose x slice is staged in LDS at once           */
  int32_t x_loads;         /* 16-byte x loads per lane and phase                      */
  int32_t row_blocks;      /* row blocks per workgroup: 1, or 4 for 8+ vectors on an  */
                           /* INT4 sparse layer with K <= 4096 and 640+ row blocks    */
                           /* (each x slice then read once for the 4 blocks)          */
  int32_t full_waves;      /* waves that take chunks_per_wave chunks (see waves)      */
} sgemv_plan_t;

/* sgemv_plan - describe the launch sgemv_run would make for (d, B) without
 * making any HIP call (for occupancy planning and host-side checks).
 * Errors: EINVAL (NULL, B outside 1..16), ESIZE (inconsistent descriptor). */
int sgemv_plan(const sgemv_desc* d, int32_t B, sgemv_plan_t* out);

/* One layer of a several-layer launch (sgemv_run_group): the arguments of
 * sgemv_run for that layer. */
typedef struct sgemv_task {
  const sgemv_desc* desc;  /* host pointer to the layer's descriptor          */
  const void* blob_dev;    /* device blob, 256-byte aligned                   */
  const void* x_dev;       /* device FP16 [B][desc->K], 16-byte aligned       */
  void* y_dev;             /* device FP16 [B][desc->N], 2-byte aligned        */
} sgemv_task;

#define SGEMV_MAX_GROUP 32

/* sgemv_run_group - several independent GEMVs y_i = W'_i x_i in one kernel
 * launch (the per-token decode of P1 §1 runs many small GEMVs back to back;
 * one launch per GEMV pays the dispatch, ramp-up and drain of a kernel each
 * time, which a 4096 x 4096 layer's few megabytes cannot hide).
 *   tasks      : host array of count layers; every layer has the same nk
 *                and value format (EINVAL otherwise); N and K may differ (workgroups of a
 *                layer with fewer column chunks than the widest one leave
 *                waves idle, so grouping layers of equal K is best).
 *   count      : 1..SGEMV_MAX_GROUP.
 *   B          : batch of every layer, 1..16.
 *   hip_stream : hipStream_t to enqueue on (NULL = default stream).
 * Results are those of sgemv_run on each layer, with the same bound; the sum
 * over column chunks may be split differently (the launch geometry follows
 * the widest layer and the summed row blocks, see sgemv_plan_group), so the
 * bits can differ from separate calls by FP32 reassociation. Outputs must
 * not overlap each other, any x or any blob. Enqueues one kernel and
 * returns without synchronising.
 * Errors: EINVAL (count, B, NULL, mixed nk), ESIZE (inconsistent descriptor
 * or sizes beyond the kernels), EALIGN, EHIP. */
int sgemv_run_group(const sgemv_task* tasks, int32_t count, int32_t B, void* hip_stream);

/* sgemv_plan_group - the launch sgemv_run_group would make (grid = summed
 * row blocks), without any HIP call. Device pointers are not examined.
 * Errors: as sgemv_run_group except EALIGN and EHIP. */
int sgemv_plan_group(const sgemv_task* tasks, int32_t count, int32_t B, sgemv_plan_t* out);

#define SGEMV_LIST_MAX 48

/* sgemv_run_list - up to SGEMV_LIST_MAX independent one-vector GEMVs
 * y_i = W'_i x_i in one kernel launch, with no workspace: the task list
 * travels in the kernel arguments. Per-token decoding runs every projection
 * of every layer as a GEMV on one vector (P1 §1 "our core idea"); one launch
 * per GEMV pays a kernel's dispatch, ramp-up and drain each time, which a
 * few megabytes of weights cannot hide.
 *   tasks      : host array of count layers in the INT4 form, each 2:4 or
 *                1:4 (they may mix), any N and K (EINVAL for the FP16-valued
 *                form or the dense ablation).
 *   count      : 1..SGEMV_LIST_MAX.
 *   B          : must be 1 (EINVAL otherwise).
 *   hip_stream : hipStream_t to enqueue on (NULL = default stream).
 * How the work is split: each layer gets workgroups of 8 waves in
 * proportion to its algorithmic bytes (up to 1536 in all, 6 per compute
 * unit of MI355X, or 3072 when the layers differ in shape or N:M choice),
 * dispatched layer by layer in order of their longest
 * wave's bytes, longest first (the order of the tasks does not matter); a
 * workgroup stages its layer's x in LDS and its waves each walk a
 * contiguous run of whole 16-row blocks, column chunk by column chunk, with
 * the loads of the next chunks in flight. Launches whose layers share one
 * shape balance best. A row's sum runs over
 * all its columns in one FP32 accumulator, so the results carry the bound
 * of sgemv_run (with n the row's kept elements); the bits can differ from a
 * separate sgemv_run by FP32 reassociation, and are the same on every call.
 * It pays off when the layers together have many row blocks per wave (a
 * decoder layer's 7 GEMVs, or more); a single layer is better served by
 * sgemv_run, which splits each row over several waves.
 * Outputs must not overlap each other, any x or any blob. Enqueues one
 * kernel and returns without synchronising.
 * Errors: EINVAL (count, B, NULL, value format), ESIZE (inconsistent
 * descriptor, or a layer whose share would exceed 256 row blocks a
 * workgroup), EALIGN, EHIP. */
int sgemv_run_list(const sgemv_task* tasks, int32_t count, int32_t B, void* hip_stream);

/* sgemv_plan_list - the launch sgemv_run_list would make, without any HIP
 * call: grid = workgroups with work, block = 64 * waves, row_blocks = the
 * most row blocks a workgroup takes, lds_bytes = LDS per workgroup (the
 * widest layer's x and a run's row indices and results). Device pointers
 * are not examined.
 * Errors: as sgemv_run_list except EALIGN and EHIP. */
int sgemv_plan_list(const sgemv_task* tasks, int32_t count, int32_t B, sgemv_plan_t* out);

#define SGEMV_LIST_TABLE_MAX 4096

/* The launch a task table describes (filled by sgemv_list_table). */
typedef struct sgemv_list_launch {
  int64_t table_bytes;     /* bytes of the table: rows * 80                          */
  int64_t lds_bytes;       /* dynamic LDS per workgroup                              */
  int64_t workgroups;      /* workgroups with work: the sum of the tasks' shares     */
  int32_t rows;            /* grid rows, one table entry each                        */
  int32_t row_width;       /* workgroups per grid row (at most 32)                   */
  int32_t tasks;           /* count                                                  */
  int32_t block;           /* lanes per workgroup (64 * 8)                           */
} sgemv_list_launch;

/* sgemv_list_table - the task list of sgemv_run_list for any number of
 * one-vector GEMVs (a whole decoder step: P1 §1 "our core idea" runs every
 * projection of every layer per token), planned once on the host into a
 * table that the caller keeps in device memory, so that one launch covers
 * them all and the per-launch ramp-up and drain are paid once.
 *   tasks       : host array of count layers, as for sgemv_run_list.
 *   count       : 1..SGEMV_LIST_TABLE_MAX.
 *   B           : must be 1 (EINVAL otherwise).
 *   table_host  : host buffer for the table, or NULL to fill *out only.
 *   table_bytes : its size; ESIZE if below out->table_bytes.
 *   out         : host pointer, the launch (grid, LDS, table size).
 * The split is that of sgemv_run_list, with 1536 (3072 for mixed shapes)
 * workgroups per 48 tasks or part of them, so each task gets the share it
 * would get in a list of 48. The table holds the tasks' device pointers and
 * their share: build it again when any of them changes. Pure host work, no
 * HIP call.
 * Errors: EINVAL (count, B, NULL, value format), ESIZE (inconsistent
 * descriptor, a share over 256 row blocks a workgroup, table too small),
 * EALIGN (a blob, x or y pointer). */
int sgemv_list_table(const sgemv_task* tasks, int32_t count, int32_t B, void* table_host,
                     int64_t table_bytes, sgemv_list_launch* out);

/* sgemv_run_list_table - enqueue the launch of a task table.
 *   table_dev  : device copy of the bytes sgemv_list_table wrote, 16-byte
 *                aligned; it must hold launch->rows entries, stay unchanged
 *                and stay allocated until the kernel has run.
 *   launch     : host pointer to the launch sgemv_list_table filled for it.
 *   hip_stream : hipStream_t to enqueue on (NULL = default stream).
 * Results are bit-for-bit those of sgemv_run_list on the same tasks (a
 * row's sum does not depend on which workgroup computes it), and the same
 * on every call. Outputs must not overlap each other, any x or any blob.
 * Enqueues one kernel and returns without synchronising.
 * Errors: EINVAL (NULL, a launch field out of range), EALIGN (table_dev),
 * EHIP. */
int sgemv_run_list_table(const void* table_dev, const sgemv_list_launch* launch, void* hip_stream);

/* sgemv_strerror - static description of a status code (never NULL). */
const char* sgemv_strerror(int code);

/* sgemv_f64_to_f16 - the packer's FP64 -> FP16 conversion, exported so that
 * callers (and tests) can reproduce the FP16 scales it stores (P1 §1 "our
 * core idea": FP16 -> INT4 compression with FP16 group scales). Round to
 * nearest, ties to even, in one step from binary64 (no intermediate FP32
 * rounding); overflow gives +-inf, values below half the smallest subnormal
 * give +-0, NaN gives the quiet NaN 0x7E00 with the input's sign.
 *   in  : host double[n];  out : host uint16_t[n] (FP16 bit patterns).
 * Errors: EINVAL (NULL with n > 0, n < 0). */
int sgemv_f64_to_f16(const double* in, uint16_t* out, int64_t n);

/* Measurement probes: the practical ceiling of one launch on this GPU, for
 * comparing sgemv_run with the cost of merely launching a kernel and of
 * merely streaming the same bytes (the pages locate the decode bottleneck
 * in weight loading: page "高效推理论文精选", section "推理瓶颈分析",
 * inference-bottleneck analysis). They compute nothing of the method.
 *
 * sgemv_probe_read - one kernel that reads `bytes` bytes at src_dev with one
 * 16-byte non-temporal load per lane (256 lanes per workgroup, grid
 * ceil(bytes / 4096)), folds each lane's 16 bytes into 4, and writes the
 * folded words of the first store_bytes / 4 lanes to dst_dev (the store of
 * a GEMV's y). Other lanes store only if their folded word equals `magic`,
 * which keeps every load live (pass a value the data is unlikely to hold;
 * such a lane writes dst_dev[0]).
 *   src_dev : device, 256-byte aligned; bytes % 16 == 0, 16 <= bytes < 2^31.
 *   dst_dev : device, 4-byte aligned, at least max(store_bytes, 4) bytes;
 *             0 <= store_bytes <= bytes / 4, store_bytes % 4 == 0.
 * sgemv_probe_empty - one kernel of `grid` workgroups of `block` lanes
 * (1..1024, a multiple of 64) whose body is empty.
 * Both enqueue on hip_stream and return without synchronising.
 * Errors: EINVAL (arguments), EALIGN, EHIP. */
int sgemv_probe_read(const void* src_dev, int64_t bytes, void* dst_dev, int64_t store_bytes,
                     uint32_t magic, void* hip_stream);
int sgemv_probe_empty(int32_t grid, int32_t block, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SGEMV_H */
