/*
 * vc.h — C ABI of the draft/verify attention library for AMD Instinct MI355X (gfx950).
 *
 * The library implements the GPU hot path of VeriCache ("VeriCache: Turning Lossy KV Cache into
 * Lossless LLM Inference", technical review page, §Draft–Verify Pipeline): a drafter decodes
 * with a compressed KV cache, a verifier attends with the full KV cache over the drafted block
 * in one parallel pass, and a greedy accept keeps the longest agreeing prefix.
 *
 * Conventions for every call
 * --------------------------
 * - Pointers marked (device) are device memory on the current HIP device; (host) are host memory.
 *   All tensors are caller-owned; the library never frees caller memory and allocates nothing
 *   except where a call says so.
 * - Calls are asynchronous on the given stream (a hipStream_t passed as void*; NULL = default
 *   stream) and never synchronise, except vc_stage_kv's event which the caller waits on.
 * - Every call validates its arguments on the host first.  On failure it returns a negative
 *   vc_status, enqueues nothing and records a message readable with vc_last_error() (per
 *   thread).  HIP errors are reported as VC_EHIP.  Nothing throws across the ABI.
 * - KV caches are paged: 16-token blocks ("pages") in a pool shared by all requests, with a
 *   per-request page table giving the physical block of each logical page; every layer of the
 *   pool uses the same table.  Positions past a request's length inside its last page, and
 *   drafted-block rows past the last visible one, may hold any bits (even NaN): they never
 *   reach a result.
 * - Page-table entries live in device memory, so the host cannot check them.  An entry of -1 is a
 *   hole (the page is absent).  An entry below -1 or at or past num_blocks is corrupt: kernels
 *   never dereference it (the page is treated as absent, or a write to it is skipped), and they
 *   record it in a per-device error word that vc_check_device() reports as VC_EDEVICE.  The word
 *   is shared by every call on the device and keeps one of the corrupt entries seen since it was
 *   last read.
 * - Shapes: head_dim d in {64, 128}; G = Hq / Hkv query heads per KV head (1..16); query head h
 *   reads KV head h / G.
 */
#ifndef VC_H
#define VC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VC_OK = 0,
  VC_EINVAL = -1,       /* bad argument; nothing was enqueued */
  VC_ENOSPACE = -2,     /* workspace too small; nothing was enqueued */
  VC_EHIP = -3,         /* a HIP runtime call failed */
  VC_EUNSUPPORTED = -4, /* valid but not implemented (e.g. head_dim 96) */
  VC_ENOMEM = -5,       /* the page allocator has too few free pages of the asked kind */
  VC_EAGAIN = -6,       /* the scheduler has no room for the request now; retry after advancing */
  VC_EDEVICE = -7       /* a kernel met a page-table entry outside [-1, num_blocks) (vc_check_device) */
} vc_status;

#define VC_BLOCK_TOKENS 16   /* tokens per KV page */
#define VC_MAX_REQS 1024     /* requests per attention launch */
#define VC_MAX_BATCH 128     /* requests per cache-building or commit call */
#define VC_MAX_ROWS 64       /* drafted rows per request */
#define VC_KIVI_GROUP 32     /* KIVI quantisation group (tokens for keys, channels for values) */

/* Page kinds of the allocator (VeriCache review, §Implementation notes, "Page table tricks"). */
#define VC_PAGE_RESIDENT 0   /* compressed-resident: allocated for the request's whole life */
#define VC_PAGE_TRANSIENT 1  /* full-transient: allocated when the full cache is reloaded */

/* Kind of work of one request in an attention launch. */
#define VC_VERIFY 0  /* x query rows, full context + causal drafted block (MFMA row tiles) */
#define VC_DRAFT 1   /* one decode step (rows*G <= 16), compressed context + drafted rows 0..q0 */

typedef struct {
  int32_t num_layers;    /* L: layer slices stored in every pool */
  int32_t num_q_heads;   /* Hq */
  int32_t num_kv_heads;  /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t max_rows;      /* XMAX: drafted-row capacity of q/blk/out tensors; multiple of 16, <= 64 */
} vc_shape;

/*
 * A paged KV pool (device memory).  nb = num_blocks, Hkv and d as in vc_shape.
 *
 * bits == 16 (bf16 cache: the full KV, or a token-dropped compact cache):
 *   k     bf16 [L][nb][Hkv][16 tokens][d]        (token-major page)
 *   v     bf16 [L][nb][Hkv][d][16 tokens]        (channel-major page)
 * bits == 2 or 4 (KIVI-style cache: keys quantised per channel over groups of 32 consecutive
 * stored tokens, values per token over groups of 32 consecutive channels; x^ = code*scale+zero):
 *   k     uint32 [L][nb][Hkv][16 tokens][d*bits/32]   codes of each token row: channel c is code
 *         u = c % (32/bits) of word c / (32/bits), stored at bit (u%2)*16 + bits*(u/2) (the two
 *         halves of a word hold the even and the odd codes, so one shift and mask yields a pair)
 *   v     uint32 [L][nb][Hkv][d][16*bits/32]          codes of each channel's 16 tokens, same
 *         packing with the token index in place of the channel
 *   k_sz  fp16 [L][nb][Hkv][2][d]   scale plane then zero plane: the (scale, zero) of each channel
 *         for the 32-token group made of logical pages 2j and 2j+1, stored in the block of page 2j
 *         (odd pages' entries unused)
 *   v_sz  fp16 [L][nb][Hkv][d/32][2][16]   per 32-channel group: the scales of the page's 16
 *         tokens, then their zeros
 * Limits: L*nb*Hkv below 2^31; in a KIVI pool also nb*Hkv*max(16*d*bits/8, 4*d) bytes (one layer
 * of the largest per-page array) below 2^32.  A launch naming a pool past them fails with
 * VC_EUNSUPPORTED before anything is enqueued.
 */
typedef struct {
  int32_t bits;                /* 16, 2 or 4 */
  int32_t max_pages;           /* row stride of page_table */
  int64_t num_blocks;          /* nb: physical blocks per layer */
  const int32_t* page_table;   /* (device) int32 [rows][max_pages]; -1 = no block.  A context
                                  page whose entry is -1 contributes no keys (one outside
                                  [-1, num_blocks) neither, and is reported as VC_EDEVICE);
                                  in a KIVI pool a missing even page 2j also removes page 2j+1
                                  (the group's key parameters live in page 2j's block) */
  const void* k;               /* (device) see above */
  const void* v;               /* (device) */
  const void* k_sz;            /* (device) KIVI only, else NULL */
  const void* v_sz;            /* (device) KIVI only, else NULL */
} vc_pool;

/*
 * One request of an attention launch.  Query rows are block positions q0 .. q0+rows-1 of request
 * slot `slot`; a row at block position j attends to ctx_len context tokens of pool `pool`
 * (logical pages from page-table row `page_row`) plus drafted-block rows 0..j.
 * Verify pass (VeriCache review, §Draft–Verify Pipeline step 4): kind VC_VERIFY, q0 = 0,
 * rows = x, the full pool.  Draft step i (steps 1–2): kind VC_DRAFT, q0 = i, rows = 1, the
 * compressed pool.
 */
typedef struct {
  int32_t slot;      /* request slot in q / blk / out (0 <= slot < batch) */
  int32_t pool;      /* index into the pools array of the call */
  int32_t ctx_len;   /* context tokens visible in that pool (>= 0) */
  int32_t page_row;  /* row of that pool's page table */
  int32_t q0;        /* block position of the first query row */
  int32_t rows;      /* query rows (>= 1); q0 + rows <= max_rows */
  int32_t kind;      /* VC_VERIFY or VC_DRAFT */
} vc_req;

/*
 * Common tensors of the attention calls (device):
 *   q      bf16 [batch][L][max_rows][Hq][d]      query of drafted-block position i at row i
 *   blk_k  bf16 [batch][L][Hkv][max_rows/16][16][d]   the drafted block's own keys (pages)
 *   blk_v  bf16 [batch][L][Hkv][max_rows/16][d][16]   and values (channel-major pages)
 *   out    fp32 [batch][L][max_rows][Hq][d]      attention output; only rows q0..q0+rows-1 of
 *          each request are written
 *   workspace: device scratch, at least vc_attn_workspace_size() bytes for the same arguments
 *          (may be NULL when that is 0): the launch's request table when it has more than 64
 *          requests (written by the call itself, on the stream, before the attention kernel),
 *          then the split-context partial results.  Calls that overlap on one workspace race.
 * Attention (VeriCache review, §Prerequisites, attention equation): softmax(q k^T / sqrt(d)) v,
 * fp32 accumulation, bf16 inputs, softmax weights rounded to bf16 for the value product.
 * split_pages: context pages per split (multiple of 4), 0 = automatic.
 */

/* Bytes of workspace an attention call with these requests needs (0 if it has at most 64
 * requests and no context is split), or 0 for arguments the call would reject. */
size_t vc_attn_workspace_size(const vc_shape* shape, int num_reqs, const vc_req* reqs /* host */,
                              int split_pages);

/* Verify pass: every request is VC_VERIFY over `full` (bf16 pool); req.pool is ignored. */
int vc_verify_attn(const vc_shape* shape, int num_reqs, const vc_req* reqs /* host */,
                   const void* q, const void* blk_k, const void* blk_v, const vc_pool* full /* host struct */,
                   float* out, void* workspace, size_t workspace_bytes, int split_pages, void* stream);

/* Draft step: every request is VC_DRAFT over `comp` (bf16 token-dropped or KIVI pool). */
int vc_draft_attn(const vc_shape* shape, int num_reqs, const vc_req* reqs /* host */,
                  const void* q, const void* blk_k, const void* blk_v, const vc_pool* comp /* host struct */,
                  float* out, void* workspace, size_t workspace_bytes, int split_pages, void* stream);

/* One launch over a mixed list: each request names its pool (0 <= pool < num_pools <= 4) and
 * kind, so drafting and verifying requests of a batch run together (VeriCache review,
 * §The two design principles, P1: every iteration mixes drafters and verifiers). */
int vc_attn_mixed(const vc_shape* shape, int num_reqs, const vc_req* reqs /* host */,
                  const void* q, const void* blk_k, const void* blk_v,
                  int num_pools, const vc_pool* pools /* host array */,
                  float* out, void* workspace, size_t workspace_bytes, int split_pages, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): vc_attn_mixed without a workspace argument.  The
 * workspace comes from a device array the library holds, VC_SCRATCH_BYTES on each device it runs
 * on, from the first call on that device until the process ends; the call allocates nothing.
 * Every output is what vc_attn_mixed writes for the same arguments.
 * Errors: as vc_attn_mixed; VC_ENOSPACE (nothing enqueued) when the launch needs more workspace
 * than VC_SCRATCH_BYTES (vc_attn_workspace_size tells; long contexts split many ways need more).
 * The array is shared by every call on a device and keeps the last call's contents (every call
 * writes what it reads, so nothing needs clearing): calls that overlap on one device (other
 * streams, other threads) race and must be ordered by the caller.
 */
#define VC_SCRATCH_BYTES (64u << 20)
int vc_attn_mixed_noalloc(const vc_shape* shape, int num_reqs, const vc_req* reqs /* host */,
                          const void* q, const void* blk_k, const void* blk_v,
                          int num_pools, const vc_pool* pools /* host array */,
                          float* out, int split_pages, void* stream);

/*
 * Greedy accept (VeriCache review, §Draft–Verify Pipeline steps 5–6) for n_inst independent
 * drafted blocks.  For instance i: x[i] drafted rows (1..max_x), xv[i] verifier rows (x[i], or
 * x[i]+1 where the extra row gives the bonus token; at most max_xv).  Logits rows are contiguous
 * over `vocab`:
 *   draft_logits  fp32 [n_inst][max_x][vocab]     row j = draft step j
 *   verify_logits fp32 [n_inst][max_xv][vocab]    row j = verifier prediction for slot j
 * Outputs (device): draft_tok int32 [n_inst][max_x], verify_tok int32 [n_inst][max_xv] (argmax,
 * ties to the lowest id; unused rows -1); accept_len int32 [n_inst] = first j < min(x, xv) with
 * draft_tok != verify_tok, else min(x, xv); next_tok int32 [n_inst] = verify_tok[accept_len] if
 * that row exists (accept_len < xv), else -1.  A verifier with fewer rows than drafted slots
 * (xv < x) thus ends the block at its last row, as in vc_accept_sampled.  x and xv are device
 * arrays (values are clamped to [0, max_x], [0, max_xv]); max_xv may be below max_x.
 * Logits must be finite.
 */
int vc_accept(int n_inst, int max_x, int max_xv, int vocab, const int32_t* x, const int32_t* xv,
              const float* draft_logits, const float* verify_logits,
              int32_t* draft_tok, int32_t* verify_tok, int32_t* accept_len, int32_t* next_tok,
              void* stream);

/*
 * Drafter-side sampling at temperature T > 0 (VeriCache review, §Implementation notes worth
 * absorbing, "Rejection sampling for non-greedy": the drafter samples its token from its own
 * distribution).  For each row r: p = softmax(logits[r] / T) in float64, and tokens[r] is the
 * smallest k with p_0 + ... + p_k > u[r] * sum(p) (inverse CDF; if rounding leaves no such k, the
 * last k with p_k > 0).
 *   logits fp32 [rows][vocab] (finite), u fp64 [rows] uniforms in (0, 1), tokens int32 [rows];
 *   all device pointers, caller-owned.  Asynchronous on `stream`.
 * Errors (nothing launched): VC_EINVAL for rows < 0, vocab < 1, T not finite and > 0, NULL.
 */
int vc_sample_tokens(int rows, int vocab, float temperature, const float* logits, const double* u,
                     int32_t* tokens, void* stream);

/*
 * Rejection-sampling accept at temperature T > 0 (VeriCache review, §Implementation notes worth
 * absorbing, "Rejection sampling for non-greedy"; the greedy rule is vc_accept).  For instance i
 * with x[i] drafted slots and xv[i] verifier rows (x[i] or x[i] + 1), slot j in order:
 *   p_lossy = softmax(draft_logits[i][j] / T), p_full = softmax(verify_logits[i][j] / T) (float64);
 *   the drafted token t = draft_tok[i][j] is kept when u_accept[i][j] * p_lossy(t) < p_full(t)
 *   (probability min(1, p_full(t) / p_lossy(t)); a t outside [0, vocab) is never kept);
 *   at the first slot not kept: accept_len[i] = j and next_tok[i] is drawn with u_resample[i][j]
 *   from max(p_full - p_lossy, 0) (from p_full if that has no mass), by the inverse CDF of
 *   vc_sample_tokens.
 * If every slot is kept: accept_len[i] = x[i], and next_tok[i] is drawn from p_full of verifier row
 * x[i] with u_resample[i][x[i]] when xv[i] = x[i] + 1, else -1.  (xv[i] < x[i] ends the block at
 * xv[i] slots.)
 *   x, xv int32 [n_inst]; draft_logits fp32 [n_inst][max_x][vocab]; verify_logits fp32
 *   [n_inst][max_xv][vocab]; draft_tok int32 [n_inst][max_x]; u_accept fp64 [n_inst][max_x];
 *   u_resample fp64 [n_inst][max_x + 1] (uniforms in (0, 1)); accept_len, next_tok int32
 *   [n_inst].  Device pointers, caller-owned; asynchronous on `stream`.
 * Errors (nothing launched): VC_EINVAL for n_inst < 0, max_x not in [1, 64], max_xv not in
 * [1, 65], vocab < 1, T not finite and > 0, NULL arguments.
 */
int vc_accept_sampled(int n_inst, int max_x, int max_xv, int vocab, float temperature, const int32_t* x,
                      const int32_t* xv, const float* draft_logits, const float* verify_logits,
                      const int32_t* draft_tok, const double* u_accept, const double* u_resample,
                      int32_t* accept_len, int32_t* next_tok, void* stream);

/*
 * LM-head stand-in used to turn attention outputs into logits: z[r][v] = sum_w o[r][w] * W_u[w][v]
 * (bf16 MFMA, fp32 accumulate; each element of o enters as two bf16 parts whose sum is within
 * 2^-18 of it, so z carries fp32 accumulation error only).  o fp32 [rows][width] with row stride ld_o floats; w_u bf16 [width][vocab];
 * z fp32 [rows][vocab].  VeriCache review, §Draft–Verify Pipeline: argmax over the logits of
 * each position.
 */
int vc_logits(int rows, int width, int vocab, const float* o, int64_t ld_o, const void* w_u,
              float* z, void* stream);

/* ---- Building caches (untimed preparation; VeriCache review, §Compression Method Integration:
 *      compress() runs once, offline, before serving).  Each call takes 1 .. VC_MAX_BATCH
 *      requests (page-table rows 0 .. batch-1); a larger batch is built by calls over row ranges.
 *      A destination page whose entry is -1 is not written. ---- */

/*
 * Write one layer of a bf16 paged pool from a dense tensor.
 * src bf16 [batch][Hkv][src_rows][d] (device): token t of request r is src[r][g][t]; only tokens
 * t < lens[r] are written (lens: host int32 [batch]); page_row of request r is r.
 * which: 0 = keys (token-major pages), 1 = values (channel-major pages).
 */
int vc_pack_bf16(const vc_shape* shape, int batch, const int32_t* lens /* host */, int layer,
                 const void* src, int64_t src_rows, const vc_pool* pool, int which, void* stream);

/*
 * Token-drop selection: for every (request r, layer l, kv head g) keep positions
 * [n_r - recent_r, n_r) plus the top_r older positions by score (larger first, ties to the lower
 * position), written ascending to kept[r][l][g][0 .. recent_r + top_r) (int32, device, row
 * stride kept_stride).  scores uint32 [batch][L][Hkv][score_stride] (device).
 * lens/recent/top: host int32 [batch] (recent, top clamped to n_r).
 */
int vc_select_kept(const vc_shape* shape, int batch, const int32_t* lens, const int32_t* recent,
                   const int32_t* top, const uint32_t* scores, int64_t score_stride,
                   int32_t* kept, int64_t kept_stride, void* stream);

/*
 * Build a compressed pool for layer range [0, L) from a bf16 source pool:
 * token j of request r in `dst` comes from source position kept[r][l][g][j] (or position j when
 * kept is NULL), for j < comp_lens[r] (host int32 [batch]).  src page_row = dst page_row = r.
 * dst->bits 16: copy (token drop).  dst->bits 2/4: KIVI-style quantisation of the gathered
 * sequence (keys per channel over groups of 32 tokens, values per token over groups of 32
 * channels; scale = fp16(RNE((max-min)/(2^b-1))), zero = fp16(RNE(min)), code =
 * clamp(RNE((x-zero)/scale), 0, 2^b-1), 0 when scale is 0; all in fp64).
 */
int vc_compress(const vc_shape* shape, int batch, const int32_t* comp_lens /* host */,
                const vc_pool* src, const int32_t* kept, int64_t kept_stride,
                const vc_pool* dst, void* stream);

/* ---- Committing accepted rows (VeriCache review, §Draft–Verify Pipeline, the per-request cycle:
 *      accepted drafted positions join the caches, rejected ones are rolled back) ---- */

/*
 * One request's commit: block rows 0 .. count-1 of request slot `slot` (the K/V of the inputs at
 * positions pos .. pos+count-1: the last accepted token and the accepted drafted tokens) are
 * appended at token positions pos .. of page-table row `page_row`.  Rows from `count` on are the
 * rejected ones; they are simply not committed (the rollback), and the block tensor is reused.
 * kept_len: for a token-drop cache, the number of kept positions before the commit (the new
 * positions pos .. pos+count-1 are appended to the kept list at kept_len ..); otherwise ignored.
 */
typedef struct {
  int32_t slot;
  int32_t pos;
  int32_t count;     /* 0 .. max_rows */
  int32_t page_row;
  int32_t kept_len;
} vc_commit;

/*
 * Append the committed block rows to a bf16 pool (the full cache): for every commit, layer and kv
 * head, block rows [0, count) go to positions [pos, pos + count) of the pool (K token-major, V
 * channel-major pages; the page-table row must already map those positions, see
 * vc_page_row_extend).  If kept is not NULL (int32 [batch][L][Hkv][kept_stride], device), the
 * positions are also appended to each (slot, layer, head) kept list at kept_len .. (token drop:
 * newly committed tokens are always kept).  blk_k / blk_v as in the attention calls.
 * Errors (nothing launched): VC_EINVAL for more than VC_MAX_BATCH commits, a non-bf16 pool,
 * counts outside [0, max_rows], or kept_len + count > kept_stride.
 */
int vc_commit_rows(const vc_shape* shape, int num, const vc_commit* commits /* host */,
                   const void* blk_k, const void* blk_v, const vc_pool* pool, int32_t* kept,
                   int64_t kept_stride, void* stream);

/*
 * vc_compress restricted to the tail of each request: storage positions from from_lens[r] on are
 * rebuilt, starting at the page (bf16 drop) or 32-token key group (KIVI) that holds from_lens[r];
 * earlier pages and groups are left as they are.  After vc_commit_rows has appended rows to the
 * full pool (and the kept lists), this brings the compressed pool up to comp_lens[r]: a KIVI key
 * group that gained tokens is re-quantised from its bf16 rows, so a group is final once its 32
 * tokens are in.  vc_compress is this call with from_lens all 0.
 */
int vc_compress_tail(const vc_shape* shape, int batch, const int32_t* from_lens /* host */,
                     const int32_t* comp_lens /* host */, const vc_pool* src, const int32_t* kept,
                     int64_t kept_stride, const vc_pool* dst, void* stream);

/* ---- Page allocator (host; VeriCache review, §Implementation notes, "Page table tricks": two
 *      page kinds per request, kept apart so that transient frees do not fragment the resident
 *      pool).  Resident blocks are ids [0, num_resident), transient ids [num_resident,
 *      num_blocks).  Not thread-safe: one allocator per caller thread. ---- */

/* Create an allocator for a pool of num_blocks blocks (*alloc = NULL on error). */
int vc_alloc_create(int32_t num_blocks, int32_t num_resident, void** alloc);
void vc_alloc_destroy(void* alloc);
/* n block ids of `kind` into ids[0..n) (host); VC_ENOMEM (nothing taken) if fewer are free. */
int vc_alloc_pages(void* alloc, int kind, int n, int32_t* ids);
/* Give n ids of `kind` back; VC_EINVAL (nothing changed) for an id that is not allocated, of the
 * other kind, out of range, or listed twice. */
int vc_alloc_release(void* alloc, int kind, int n, const int32_t* ids);
/* Free ids of `kind`, or -1 for a bad argument. */
int32_t vc_alloc_free_count(const void* alloc, int kind);
/* Grow one request's host page-table row from old_len to new_len tokens: blocks of `kind` for the
 * logical pages that new_len adds (VC_ENOMEM, nothing changed, if short). */
int vc_page_row_extend(void* alloc, int kind, int32_t* row, int32_t max_pages, int32_t old_len,
                       int32_t new_len);
/* Shrink a row from old_len to new_len tokens: the pages no longer needed are released and their
 * entries set to -1 (a rollback past a page boundary, or freeing a transient full cache). */
int vc_page_row_truncate(void* alloc, int kind, int32_t* row, int32_t max_pages, int32_t old_len,
                         int32_t new_len);

/* ---- Admit scheduler (host; VeriCache review, §Runtime Algorithm Deep Dive: resource model,
 *      Admit, execution loop).  A window of W future iterations and two reserve rings: the link
 *      time of full-cache reloads per window (at most t_iter: the link is serial) and the bytes
 *      of full caches in HBM per window (at most hbm_budget).  A reload lasts
 *      l = KV_full / (link_bw * t_iter) iterations and occupies S = max(1, ceil(l)) windows ending
 *      at the request's verify; its link time is spread evenly over them and its KV_full counts in
 *      HBM for all of them.  Not thread-safe. ---- */

typedef struct {
  int32_t window;       /* W: lookahead iterations, >= 2 */
  int32_t draft_len;    /* x: the ideal draft length (verify slot searched outward from it) */
  double t_iter;        /* expected seconds per iteration, > 0 */
  double link_bw;       /* host-link bytes per second, > 0 */
  double hbm_budget;    /* bytes of HBM for full caches in flight, >= 0 */
} vc_sched_cfg;

int vc_sched_create(const vc_sched_cfg* cfg, void** sched);
void vc_sched_destroy(void* sched);
/* Admit(req): try verify slots d = x, x+1, x-1, x+2, ... within [S, W-1] (relative to the current
 * iteration) and reserve the first span [d-S+1, d] that fits both rings; *verify_iter = the
 * absolute iteration of the verify.  VC_EAGAIN (*verify_iter = -1, nothing reserved) when no span
 * fits now; VC_EINVAL if req already holds a reservation. */
int vc_sched_admit(void* sched, int32_t req, double kv_full_bytes, int64_t* verify_iter);
/* End the current iteration: reservations whose verify was this iteration end, the window slides. */
int vc_sched_advance(void* sched);
/* The current iteration (0 after create), or -1 for NULL. */
int64_t vc_sched_now(const void* sched);
/* Reserved link seconds and HBM bytes of window i (0 = the current iteration). */
int vc_sched_ring(const void* sched, int32_t i, double* link_s, double* hbm_bytes);
/* Requests whose reload starts at the current iteration and requests that verify at it (ascending
 * ids, at most cap of each; VC_EINVAL if more). */
int vc_sched_due(const void* sched, int32_t cap, int32_t* reload_ids, int32_t* n_reload,
                 int32_t* verify_ids, int32_t* n_verify);

/* ---- Staging the full KV into HBM (VeriCache review, §KV Swap Scheduling: the full cache is
 *      reloaded from host memory ahead of its verify, overlapped with drafting) ---- */

/*
 * Copy `bytes` from pinned host memory (allocated with hipHostMalloc or equivalent) to device
 * memory on `side_stream`, then record `event` (a hipEvent_t as void*, may be NULL) on it; the
 * event is recorded for bytes == 0 too.  The caller makes its verify stream wait on the event.
 * Nothing is synchronised here.
 * Errors (nothing enqueued): VC_EINVAL for NULL pointers with bytes > 0, a source that is not
 * pinned host memory (a pageable source would make the copy synchronous, so the staging would no
 * longer overlap the draft steps), or a destination that is not device memory.
 */
int vc_stage_kv(void* dst_device, const void* src_pinned_host, size_t bytes, void* side_stream,
                void* event);

/*
 * Report the device-side checks of earlier calls on the current device.  Synchronises `stream`
 * (a hipStream_t as void*, NULL = the null stream), reads the device error word and clears it.
 * Returns VC_OK, or VC_EDEVICE with the page-table row, logical page and entry of one corrupt
 * page-table entry in vc_last_error().  Work still running on other streams may report later.
 * This is the one call of the library that waits for the device.
 */
int vc_check_device(void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* vc_last_error(void);

/* Library version, e.g. "vc 0.1 gfx950". */
const char* vc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VC_H */
