/*
 * paged_attn.h - C ABI of the MI355X (gfx950) paged GQA decode-attention
 * library (libpaged_attn.so).
 *
 * The operation is one decode step of grouped-query attention over a paged
 * K/V pool, as the lucebox PR #555 page states it (Summary): a single query
 * token per sequence, Hq query heads sharing Hkv K/V heads, K/V rows reached
 * through a per-sequence table of fixed-size blocks, F16, Q8_0 or Q4_0 K and V
 * (chosen independently), the context of each sequence split into partitions
 * whose partial results are recombined by a max-shifted merge of their
 * softmax sums. For each sequence b and query head h, with r = Hq/Hkv, kv head
 * g = h / r and L = seq_len[b]:
 *
 *     out[b,h,:] = sum_t softmax_t(scale * q[b,h,:] . K[b,g,t,:]) V[b,g,t,:]
 *
 * over t < L (a zero row when L == 0).
 *
 * Conventions for every call
 *   - All tensors live in device memory owned by the caller; the library
 *     allocates no device memory and keeps no state across calls beyond the
 *     cached device properties and the caller's kv_pool objects.
 *   - GPU work is enqueued on the caller's stream (`stream` is a hipStream_t,
 *     NULL = the null stream) and is asynchronous; results are valid once the
 *     stream has reached that point.
 *   - Host-detectable problems return a negative PA_ERR_* code synchronously
 *     and enqueue nothing; pa_last_error() then returns a message that names
 *     the entry point (the mlxcel issue #2153 page, Proposed Solution: a
 *     refused launch reports the entry point instead of computing garbage).
 *   - Pools are addressed with 64-bit byte offsets everywhere, so a pool side
 *     may hold more than 2^32 elements (mlxcel issue #2153, Problem and
 *     Proposed Solution: a row's offset, block id times block size plus
 *     slot, times the token stride, plus the head's offset, is formed in
 *     64-bit arithmetic before any product; a pool of exactly 2^32 elements
 *     addresses its last element). There is no size refusal for
 *     large pools.
 *
 * Layouts (row-major, little endian)
 *   q          float32 [B, Hq, D]
 *   out        float32 [B, Hq, D]
 *   k_pool     uint8   [nblocks, block_size, Hkv, row_bytes(k_type, D)]
 *   v_pool     uint8   [nblocks, block_size, Hkv, row_bytes(v_type, D)]
 *   block_table int32  [B, max_blocks]: physical block of each logical block;
 *              only entries j < ceil(seq_len[b]/block_size) are ever read.
 *   seq_len    int32   [B] (device memory)
 *   One row holds the D values of one (token slot, kv head):
 *     PA_F16  : D IEEE binary16 values                      (2*D bytes)
 *     PA_Q8_0 : D/32 blocks {f16 d; int8 q[32]}, x = d*q    (34*D/32 bytes)
 *     PA_Q4_0 : D/32 blocks {f16 d; uint8 n[16]}; element j of a block is
 *               (n[j] & 15) - 8, element j+16 is (n[j] >> 4) - 8, times d
 *                                                           (18*D/32 bytes)
 *
 * Supported shapes: D in {128, 256}; r = Hq/Hkv integral, 1 <= r <= 16;
 * block_size a power of two in [16, 256]; 1 <= B <= 1024. Others return
 * PA_ERR_UNSUPPORTED ("unsupported combinations fail explicitly", lucebox
 * PR #555, Scope).
 *
 * Numerics: q is rounded to f16 after the softmax scale (and log2 e) is folded
 * in; dequantised K/V values are rounded to f16; dot products, softmax and
 * accumulation run in fp32. Live K/V values must lie inside the f16 range
 * (true for any Q8_0/Q4_0 block quantised from f16-range data).
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* K/V element formats (nine K/V pairs: lucebox PR #555, Validation). */
enum { PA_F16 = 0, PA_Q8_0 = 1, PA_Q4_0 = 2 };

/* Return codes. */
enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,      /* null pointer, inconsistent shape, ws too small, bad argument */
  PA_ERR_UNSUPPORTED = -2,  /* a shape/type combination this build does not compile */
  PA_ERR_CAPACITY = -3,     /* kv_pool: not enough free blocks (state unchanged) */
  PA_ERR_STALE_HANDLE = -4, /* kv_pool: released, double-released or pre-reset handle */
  PA_ERR_HIP = -5           /* a HIP runtime call failed */
};

/* Bits of the device status word (see paged_attn_status). */
enum {
  PA_STATUS_BAD_BLOCK_ID = 1, /* a live table entry was < 0 or >= nblocks; that
                                 sequence's output rows are NaN */
  PA_STATUS_BAD_SEQ_LEN = 2,  /* seq_len[b] < 0 or longer than the plan admits
                                 (min(max_blocks*block_size, p_max*psize), at
                                 least plan->max_seq_len); it was clamped into
                                 range */
  PA_STATUS_MERGE_WAIT = 4    /* single-launch merge: a merge slice found its
                                 completion counter past the partition count
                                 (counters not zero at the call) or waited
                                 longer than one second; its 64 columns are
                                 NaN */
};

typedef struct pa_shape {
  int32_t B;          /* sequences in the batch */
  int32_t Hq;         /* query heads */
  int32_t Hkv;        /* K/V heads; Hq % Hkv == 0 */
  int32_t D;          /* head dimension */
  int32_t block_size; /* token slots per block */
  int32_t nblocks;    /* blocks in each pool */
  int32_t max_blocks; /* columns of the block table */
  int32_t k_type;     /* PA_F16 / PA_Q8_0 / PA_Q4_0 */
  int32_t v_type;
} pa_shape;

/* A decode plan: fixed launch geometry and workspace size for one shape.
 * Produced by paged_attn_plan; treat as read-only. */
typedef struct pa_plan {
  pa_shape shape;
  float scale;          /* softmax scale applied to q.k */
  int32_t psize;        /* tokens per context partition (multiple of 32) */
  int32_t p_max;        /* partitions of the longest admissible sequence */
  int32_t max_seq_len;  /* longest seq_len the plan admits */
  int32_t grid;         /* workgroups launched by paged_attn_decode */
  int32_t num_cus;      /* compute units the plan was sized for */
  int32_t direct;       /* 1: p_max == 1, decode writes out, merge is a no-op */
  int32_t path;         /* decode kernel: 2 = LDS-staged (K/V blocks DMA'd into
                           LDS, one workgroup per 4 kv heads; needs Hkv % 4 == 0,
                           B <= 256, and pools and q 16-byte aligned, else
                           path 1 runs), 1 = register-streaming.
                           paged_attn_plan picks 2 where the shape allows it; a
                           caller may set 1 to force the register kernel (and
                           must then set fused = 0). The two kernels differ
                           only in the order of fp32 accumulation. */
  int32_t fused;        /* 1: single launch - the LDS-staged decode kernel also
                           merges the partials (its last workgroups to finish
                           take the merge slices once their partitions are in,
                           counted by atomic completion counters in ws:
                           llama.cpp PR #13 HRX, Changes: the partials reduced
                           by the decode launch itself; lucebox PR #555,
                           Roadmap item 4) and paged_attn_merge is a no-op.
                           Allowed on path 2 when not direct and the merge is
                           of the wide layout (not the row-per-thread one).
                           paged_attn_plan leaves it 0: on MI355X the separate
                           merge launch measured faster at every shape tried.
                           Both give the same bits. */
  int32_t reserved;     /* 0 */
  uint64_t ws_bytes;    /* workspace bytes paged_attn_decode/merge need */
  uint64_t part_offset; /* byte offset of the partials in ws (see layout) */
} pa_plan;

/* Bytes of one encoded row of D values of `type`, or a negative PA_ERR_*. */
int32_t pa_row_bytes(int32_t type, int32_t D);

/* Message of the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

/*
 * paged_attn_plan - choose the context partitioning and launch geometry.
 *
 * The partition size follows the lucebox PR #555 page (Summary:
 * occupancy-aware context partitioning): it is sized from the number of
 * compute units and the work in the batch, never below the size at which the
 * partial-result traffic would exceed a few percent of the K/V bytes.
 *   max_seq_len      longest seq_len any later decode with this plan will see
 *                    (<= max_blocks*block_size)
 *   total_tokens     sum of seq_len over the batch if known (sizes the grid for
 *                    ragged batches); 0 = assume B*max_seq_len. Only speed
 *                    depends on it: every live partition is processed for any
 *                    value.
 *   num_cus          compute units to size for; 0 = query the current device
 *   force_partitions 0 = automatic; 1 = direct mode (one partition, no merge:
 *                    the lucebox page's forced single partition); n > 1 = at
 *                    most n partitions of equal size for the longest sequence
 *   partition_tokens 0 = automatic, else the exact partition size (rounded up
 *                    to a multiple of 32); overrides force_partitions
 *   scale            softmax scale; 0 = 1/sqrt(D)
 * Returns PA_OK and fills *plan, or a negative code.
 */
int32_t paged_attn_plan(const pa_shape* shape, int32_t max_seq_len, int64_t total_tokens,
                        int32_t num_cus, int32_t force_partitions, int32_t partition_tokens,
                        float scale, pa_plan* plan);

/*
 * Workspace layout (ws, plan->ws_bytes bytes, device memory, 256-byte aligned):
 *   [0, 4)      uint32 status word (PA_STATUS_* bits); must be zero before the
 *               first decode; paged_attn_status reads and clears it
 *   [4, 12)     uint32 item counter and leave counter of the single-launch
 *               merge (plan->fused)
 *   [12, 256)   reserved
 *   [256, part_offset)
 *               uint32 done[B*ceil(Hkv/4)], one every 1040 words (4160 bytes):
 *               partitions finished per (sequence, kv-head quad), for the
 *               single-launch merge
 *               The counters [4, 12) and done[] must be zero before the first
 *               fused decode (the workspace is zero-filled once); every fused
 *               decode leaves them zero (its last workgroup resets them), and
 *               no call of the same B and Hkv writes them. A plan of a smaller
 *               B or Hkv has a smaller part_offset and writes partials there:
 *               zero the workspace again before a fused decode that follows
 *               such a plan on it. Calls that share one workspace must not
 *               overlap in time.
 *   partials    only when plan->direct == 0, at offset plan->part_offset
 *               (256 + 4160*B*ceil(Hkv/4) rounded up to 256):
 *               uint16 o[B][Hq][p_max][D]  normalised output of each partition
 *                                          as IEEE binary16, rounded to nearest
 *                                          even (lucebox PR #555, Summary:
 *                                          normalised f16 partials; |o| never
 *                                          exceeds the largest |V| value)
 *               float ml[B][Hq][p_max][2]  at offset part_offset + 2*B*Hq*p_max*D:
 *                                          (m, l): m is a reference value of
 *                                          the base-2 logits x = log2(e)*scale*q.k
 *                                          of the partition with
 *                                          m <= max x <= m + 8 (the kernel moves
 *                                          its reference only when a logit
 *                                          exceeds it by more than 8),
 *                                          l = sum of 2^(x - m)
 *               Partition p of sequence b covers tokens [p*psize,
 *               min(seq_len, (p+1)*psize)); only p < ceil(seq_len/psize) is
 *               written or read. A partition that met a bad block id holds
 *               NaN in m.
 */

/*
 * paged_attn_decode - attention of one decode step over the paged pool.
 *
 * Computes, for every live (sequence, K/V head, partition), the partial
 * softmax statistics and normalised partial output of all r query heads of the
 * group from one pass over the partition's K/V rows (lucebox PR #555, Summary:
 * each K/V row read once serves every query head that shares it, base-2
 * softmax, partials kept normalised; mlxcel issue #2153: 64-bit pool
 * offsets). In direct mode
 * writes out[] instead of partials.
 *   q, k_pool, v_pool, seq_len, out: as in the layout table above
 *   block_table  NULL selects the contiguous layout: sequence b's logical
 *                block j is physical block b*max_blocks + j (computed, not
 *                read; the TensorFold PR #1418 page's null page table). The
 *                same plan then gives bit-identical results to a table that
 *                names the same rows.
 *   ws, ws_bytes workspace of at least plan->ws_bytes bytes
 *   out          written only in direct mode (may be NULL otherwise)
 * Results are deterministic: fixed reduction order, no floating-point atomics.
 * A live table entry outside [0, nblocks) is never dereferenced: the status
 * bit is set and the rows of that sequence become NaN.
 */
int32_t paged_attn_decode(const pa_plan* plan, const float* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_table,
                          const int32_t* seq_len, void* ws, uint64_t ws_bytes, float* out,
                          void* stream);

/*
 * paged_attn_merge - max-shifted merge of the partition partials in ws.
 *
 * For each (b, h) over its live partitions p < ceil(seq_len[b]/psize):
 *   M = max_p m_p;  w_p = 2^(m_p - M) * l_p;  out = sum_p w_p o_p / sum_p w_p
 * (lucebox PR #555, Summary; llama.cpp PR #13 HRX, Changes: per-block
 * normalisation scale). seq_len = 0 gives a zero row; a NaN m gives a NaN
 * row. A no-op returning PA_OK in direct mode.
 */
int32_t paged_attn_merge(const pa_plan* plan, const void* ws, uint64_t ws_bytes,
                         const int32_t* seq_len, float* out, void* stream);

/*
 * paged_attn_step - one whole decode step: paged_attn_decode followed by
 * paged_attn_merge on the same stream (lucebox PR #555, Summary: a decode
 * step attends over context partitions whose partials are then recombined by
 * the split-softmax merge). Arguments, ownership and errors as for the two
 * calls; the first refusal is returned and nothing after it is launched.
 */
int32_t paged_attn_step(const pa_plan* plan, const float* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_table,
                        const int32_t* seq_len, void* ws, uint64_t ws_bytes, float* out,
                        void* stream);

/*
 * paged_attn_step_noalloc - paged_attn_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same decode + merge kernels, with the workspace
 * in a static device array of 64 MiB per GPU that the library holds from its
 * load until the process ends, instead of a caller-provided ws. The caller
 * still passes q, the pools, the table, seq_len and out, laid out as for
 * paged_attn_step; the call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine) and enqueues nothing but the kernels.
 *   Returns PA_ERR_INVALID when plan->ws_bytes exceeds the 64 MiB scratch or
 *   plan->fused is set (the single launch needs counters that start at zero,
 *   and in the shared scratch a two-launch plan of a smaller batch writes its
 *   partials where they lie), PA_ERR_HIP when the scratch's device address
 *   cannot be obtained, else as paged_attn_step.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap on one
 *   GPU (other streams, other host threads) race and must be serialised by the
 *   caller. The scratch's status word is not readable: a corrupt block table
 *   shows only as NaN rows of the sequence concerned, and a clamped seq_len
 *   not at all (use paged_attn_step with a workspace to read the status).
 */
int32_t paged_attn_step_noalloc(const pa_plan* plan, const float* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_table,
                                const int32_t* seq_len, float* out, void* stream);

/*
 * paged_kv_gather - copy raw encoded rows out of a pool through the table,
 * with the same 64-bit address computation the decode kernel uses (the
 * mlxcel issue #2153 page, Scope: the gather path).
 *   pool      k_pool (which = 0, row format k_type) or v_pool (which = 1)
 *   b, t0, n  rows of tokens t0 .. t0+n-1 of sequence b; requires
 *             0 <= t0, t0+n <= max_blocks*block_size and every table entry
 *             they touch inside [0, nblocks) (checked on the device: rows
 *             behind a bad entry are left untouched and the status bit is set)
 *   dst       uint8 [n, Hkv, row_bytes]
 *   ws        workspace whose status word records bad entries (may be NULL)
 */
int32_t paged_kv_gather(const pa_plan* plan, const void* pool, int32_t which,
                        const int32_t* block_table, int32_t b, int32_t t0, int32_t n, void* dst,
                        void* ws, void* stream);

/*
 * paged_attn_status - synchronise `stream`, then read and clear the status
 * word of ws into *flags (PA_STATUS_* bits). The word is how the kernels
 * report what only the device sees: a live block-table entry outside the
 * pool or a seq_len outside the table's capacity (lucebox PR #555,
 * Validation: bounds guards on corrupt block tables). ws is the workspace
 * the decode, chunk or gather calls were given (its first 4 bytes).
 * Returns PA_ERR_INVALID for null arguments and PA_ERR_HIP if the copy or
 * the synchronisation fails; *flags is then unchanged.
 */
int32_t paged_attn_status(void* ws, void* stream, uint32_t* flags);

/*
 * Multi-token queries over the paged pool: chunked prefill and verify windows
 * (lucebox PR #555, Roadmap item 3: several query tokens per sequence attend
 * over the K/V already in the pool, causally inside the chunk; TensorFold PR
 * #1418, What: paged prompt-chunk attention equal to the contiguous one).
 *
 * q and out are fp32 [B][Tq][Hq][D]. seq_len[b] = L counts the chunk's own
 * tokens, whose K/V rows are already in the pool as the last Tq of the
 * sequence: chunk token t sits at position L - Tq + t and attends to the keys
 * at positions 0 .. L - Tq + t of kv head h / (Hq/Hkv). A sequence with L = 0
 * gives zero rows; 0 < L < Tq also gives zero rows and sets
 * PA_STATUS_BAD_SEQ_LEN. The key range is cut into partitions whose
 * partials (the decode layout with Tq*Hq rows per sequence) are reduced by
 * the same max-shifted merge; one partition writes out directly.
 * Three kernels compute it: path 1 converts each key/value tile once per
 * workgroup into LDS for four waves of 16 query rows (any Tq); path 2, for
 * Tq*Hq/Hkv <= 32 query rows per kv head at D = 256 (48 at D = 128, and at
 * D = 256 with Q4_0 K and V) with Hkv a multiple of 4 (verify windows),
 * streams the pool through the decode kernel's LDS ring, each wave serving
 * one kv head with all of its rows (at D = 256 with more than 16 rows, two
 * waves per kv head, each over half of the head dimension, adding their
 * partial scores through LDS); path 3, for more than 64 query rows per kv
 * head (prefill chunks), converts each tile once per workgroup for 128 query
 * rows on 32x32 MFMAs, in eight waves (score waves and conversion waves two
 * per SIMD) or, for F16 K and V at D = 256 and F16 with Q8_0, in four (there
 * the plan takes it only where its units fill at least half the compute
 * units). The plan picks path 2 or 3 where it applies; a caller may
 * set path = 1 on any plan, or 3 on one for path 1, to force that kernel.
 * Pools or q that are not 16-byte aligned (or a ws that is not, outside
 * the layout above) run path 1.
 */
typedef struct pa_chunk_plan {
  pa_shape shape;
  int32_t tq;           /* query tokens per sequence (1 .. 4096) */
  float scale;          /* softmax scale applied to q.k */
  int32_t psize;        /* keys per partition (multiple of 32) */
  int32_t p_max;        /* partitions of the longest admissible sequence */
  int32_t max_seq_len;
  int32_t grid;         /* workgroups (four wave64s each) */
  int32_t num_cus;
  int32_t direct;       /* 1: one partition, no merge */
  int32_t path;         /* 1: tile-conversion kernel, 2: window kernel,
                           3: wide-tile kernel */
  uint64_t ws_bytes;    /* workspace: header + partials (part_offset +
                           B*Tq*Hq*p_max*(2D+8) bytes when direct == 0) */
  uint64_t part_offset; /* byte offset of the partials in ws: the decode
                           layout's (the header and done[] counters are left
                           alone, so one workspace may serve both) */
} pa_chunk_plan;

/* Plan a chunk launch; arguments as for paged_attn_plan plus tq (the number
 * of query tokens per sequence). total_tokens = 0 assumes B*max_seq_len. */
int32_t paged_attn_chunk_plan(const pa_shape* shape, int32_t tq, int32_t max_seq_len,
                              int64_t total_tokens, int32_t num_cus, int32_t force_partitions,
                              int32_t partition_tokens, float scale, pa_chunk_plan* plan);

/* One chunk step: the chunk kernel, then the merge when direct == 0
 * (stream-ordered, allocates nothing). Argument rules as for
 * paged_attn_decode; q, out: fp32 [B][Tq][Hq][D]. */
int32_t paged_attn_chunk(const pa_chunk_plan* plan, const float* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_table, const int32_t* seq_len,
                         void* ws, uint64_t ws_bytes, float* out, void* stream);

/*
 * paged_table_update - write a few entries of the device-resident block table
 * and seq_len (lucebox PR #555, Summary: the table and lengths live on the
 * device beside the pool, so a step sends only the ids of newly allocated
 * blocks rather than re-sending the table).
 *   table       device int32 [B][max_blocks]; seq_len device int32 [B]
 *   updates     HOST int32 [n][3] triples (b, slot, value): slot >= 0 sets
 *               table[b][slot] = value, slot == -1 sets seq_len[b] = value.
 *               Read before the call returns (they travel in the kernel
 *               arguments), so the array may be reused at once.
 *   n           >= 0 (0 is a no-op); any number, launched 256 per kernel
 * Stream-ordered; allocates nothing. PA_ERR_INVALID (nothing launched) for
 * b outside [0, B), slot outside [-1, max_blocks) or two triples naming the
 * same entry. Values are not checked here: decode checks every block id it
 * reads and clamps seq_len (status bits).
 */
int32_t paged_table_update(int32_t* table, int32_t* seq_len, int32_t B, int32_t max_blocks,
                           const int32_t* updates, int32_t n, void* stream);

/*
 * paged_kv_copy_blocks - copy whole blocks inside one pool: the device half
 * of copy-on-write (lucebox PR #555, Roadmap item 6: prefix blocks shared
 * under reference counts and copied on write). After kv_pool_cow hands an
 * allocation a private id for a shared block, copy the shared block there
 * (in the K pool and in the V pool) before writing into it.
 *   pool          device memory, 16-byte aligned: nblocks blocks of
 *                 block_bytes = block_size*Hkv*row_bytes bytes (a multiple
 *                 of 16)
 *   src_ids, dst_ids  HOST int32 [n]: block src_ids[i] is copied to
 *                 dst_ids[i]; read before the call returns
 * Stream-ordered; allocates nothing. PA_ERR_INVALID (nothing launched) for
 * ids outside [0, nblocks), a block that is both a source and a destination,
 * or a destination named twice.
 */
int32_t paged_kv_copy_blocks(void* pool, uint64_t block_bytes, int32_t nblocks,
                             const int32_t* src_ids, const int32_t* dst_ids, int32_t n,
                             void* stream);

/*
 * Fixed-block allocator over the block ids [0, nblocks) of a caller-owned
 * pool (lucebox PR #555, Summary and Validation: an allocation either gets all
 * of its blocks or none, a freed or reset handle is refused when used again,
 * blocks return to the pool at once, and the pool resets between requests).
 * Host only; thread-safe per pool object.
 *
 * An allocation is a list of block ids, in the order they were handed out,
 * named by a 64-bit handle (slot index and generation; 0 is never a valid
 * handle). Any use of a handle that was released, released twice or issued
 * before a reset returns PA_ERR_STALE_HANDLE and changes nothing.
 *
 * Prefix sharing (lucebox PR #555, Roadmap item 6: prefix blocks shared under
 * reference counts and copied on write): every block counts the allocations
 * that hold it. kv_pool_fork starts an allocation with another's first
 * blocks; a block goes back to the pool the moment the last allocation
 * holding it is released; kv_pool_cow gives an allocation a private block in
 * place of a shared one before it writes there.
 */
typedef struct kv_pool kv_pool;

int32_t kv_pool_create(int32_t nblocks, kv_pool** pool);
int32_t kv_pool_destroy(kv_pool* pool);

/* Append n blocks to the allocation *handle (0 = open a new one and store its
 * handle). All or nothing: with fewer than n free blocks returns
 * PA_ERR_CAPACITY and leaves the pool and *handle unchanged. Writes the n new
 * ids to ids_out (may be NULL when n == 0). */
int32_t kv_pool_alloc(kv_pool* pool, int32_t n, int32_t* ids_out, uint64_t* handle);

/* Return every block of the allocation to the pool; the handle goes stale. */
int32_t kv_pool_release(kv_pool* pool, uint64_t handle);

/* Return every block; every handle issued so far goes stale. */
int32_t kv_pool_reset(kv_pool* pool);

/* Free blocks (>= 0) or a negative code. */
int32_t kv_pool_free_count(const kv_pool* pool);

/* Blocks held by an allocation (>= 0) or a negative code. */
int32_t kv_pool_count(const kv_pool* pool, uint64_t handle);

/* Copy up to cap ids of an allocation, in order, to ids_out; returns the
 * number held (may exceed cap) or a negative code. */
int32_t kv_pool_blocks(const kv_pool* pool, uint64_t handle, int32_t* ids_out, int32_t cap);

/* Open a new allocation (*handle) holding the first n_shared blocks of the
 * live allocation src (0 <= n_shared <= its block count); each of those blocks
 * gains a reference. Grow it with kv_pool_alloc as usual. */
int32_t kv_pool_fork(kv_pool* pool, uint64_t src, int32_t n_shared, uint64_t* handle);

/* Make block `index` of an allocation private before writing into it. If no
 * other allocation holds it: *id_out = that id, *copy_from = -1 (write in
 * place). Otherwise a free block replaces it in this allocation (the shared
 * block loses a reference): *id_out = the new id, *copy_from = the shared id,
 * whose bytes the caller copies over with paged_kv_copy_blocks. With no free
 * block returns PA_ERR_CAPACITY and changes nothing. */
int32_t kv_pool_cow(kv_pool* pool, uint64_t handle, int32_t index, int32_t* id_out,
                    int32_t* copy_from);

/* Allocations holding block id (0 = free) or a negative code. */
int32_t kv_pool_refcount(const kv_pool* pool, int32_t id);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
