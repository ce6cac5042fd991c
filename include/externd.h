/*
 * externd.h — C ABI of the MI355X (gfx950) ExTernD library.
 *
 * ExTernD ("ExTernD: Expanded-Rank Ternary Decomposition Ternary LLM PTQ with
 * Accuracy Approaching Any Quantization Level") approximates a real matrix
 * A (m x n) by B diag(D) C with ternary B (m x k), ternary C (k x n) and real
 * D (k), k = mu * min(m, n) (§2.1).  Component i is fitted to the residual
 * R = A - sum_{j<i} d_j b_j c_j^T by a fixed number of alternating ternary fits
 * v = T_tau(R^T u), u = T_tau(R v) (§2.3 step 1, T_tau of §2.2), given the
 * least-squares scale d = u^T R v / (|u|^2 |v|^2) (§2.3 step 2) and deflated
 * out of R (§2.3 step 3).  Block mode extracts b components at a time with
 * decorrelated targets and a joint scale solve (§2.4).
 *
 * Conventions for every entry point:
 *  - Pointers named A, R, x, y, B2, C2, D, energy, trace, stats, capture_* and
 *    workspace are DEVICE pointers (hipMalloc'd or equivalent) on the current
 *    HIP device.  The caller owns every buffer; the library never frees them.
 *  - Matrices are row-major and densely packed (leading dimension = columns).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    All device work is enqueued on it; entry points return without waiting
 *    for it, so device outputs are valid once the stream has completed.
 *  - Argument errors are detected on the host before anything is enqueued
 *    and return EXTERND_EINVAL; device-side failures return EXTERND_EHIP with
 *    a message available from externd_last_error().
 *  - 2-bit ternary codes: a row of length L occupies ceil(L/16) uint32 words;
 *    element j sits in bits 2*(j%16)..2*(j%16)+1 of word j/16 with
 *    00 = 0, 01 = +1, 11 = -1 (10 never produced).  Padding bits are 00.
 *    B2 is component-major: row i (ceil(m/16) words) holds column i of B.
 *    C2 row i (ceil(n/16) words) holds row i of C.
 */
#ifndef EXTERND_H
#define EXTERND_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum externd_status {
  EXTERND_OK = 0,
  EXTERND_EINVAL = 1,       /* bad argument (null pointer, size, non-finite knob) */
  EXTERND_ENOMEM = 2,       /* workspace allocation failed or too small */
  EXTERND_EHIP = 3,         /* HIP runtime error or a failed kernel launch */
  EXTERND_EUNSUPPORTED = 4  /* device is not gfx950 / shape outside a mode's limits */
};

/* Execution modes of the sequential path. */
enum externd_mode {
  EXTERND_MODE_AUTO = -1,      /* resident when the shape fits on chip, else persistent streaming
                                  when it applies, else streaming */
  EXTERND_MODE_STREAMING = 0,  /* R in device memory, a few kernels per ALS half-step */
  EXTERND_MODE_RESIDENT = 1,   /* one cooperative kernel, R kept in LDS/VGPRs */
  EXTERND_MODE_PERSISTENT = 2  /* one cooperative kernel, R in device memory: n % 4 == 0,
                                  m, n <= 10240 and at most 64 rows per CU; not with the
                                  optimal projection or an applied safeguard */
};

enum externd_ternarizer { EXTERND_TERN_MEAN = 0, EXTERND_TERN_PROJECTION = 1 };

/* Indices into the optional int64 statistics array (EXTERND_STATS_LEN entries). */
enum externd_stat {
  EXTERND_STAT_SUM_NNZ_U = 0,   /* sum over components and iterations of nnz(u_t) */
  EXTERND_STAT_SUM_NNZ_V = 1,   /* same for v_t */
  EXTERND_STAT_NNZ_B = 2,       /* nonzeros in the final B */
  EXTERND_STAT_NNZ_C = 3,       /* nonzeros in the final C */
  EXTERND_STAT_FALLBACKS = 4,   /* T_tau calls that fell back to the single largest entry */
  EXTERND_STAT_NONFINITE = 5,   /* non-finite entries found in A (energy is NaN if > 0) */
  EXTERND_STAT_MODE = 6,        /* mode actually run (0 streaming, 1 resident, 2 block,
                                   3 persistent streaming) */
  EXTERND_STAT_GRID = 7,        /* workgroups of the resident or persistent kernel (0 otherwise) */
  EXTERND_STAT_RIDGE_RETRIES = 8, /* block mode: joint scale solves retried with a ridge */
  EXTERND_STAT_TIMEOUTS = 9,    /* waits that ran out (energy is NaN): resident exchange, or
                                   block mode's Gram-before-inverse wait */
  EXTERND_STAT_INVERSE_UNCONVERGED = 10, /* block mode, b <= 64: Gram inverses whose fp64
                                    residual ||I - (G + eps I) X||_F stayed at or above 1e-3
                                    after the fp64 refinement (the inverse is then not known
                                    to 1e-6); wider blocks invert exactly in fp64: always 0 */
  EXTERND_STAT_SWEEP_KEPT_OLD = 11, /* block mode: sweep visits that kept the stored block */
  EXTERND_STAT_NS_ITERATIONS = 12,  /* block mode, b <= 64: Newton-Schulz residual evaluations over all Gram inverses */
  EXTERND_STAT_NS_RESTARTS = 13,    /* block mode, b <= 64: warm starts replaced by another start */
  EXTERND_STAT_ITERATIONS = 14,     /* ALS iterations run, over all components (blocks) */
  EXTERND_STAT_SAFEGUARD = 15,      /* components (sequential) or blocks (block mode) whose
                                       decrease of ||R||^2 fell below the single-entry bound
                                       max_ij w_j R_ij^2 of the residual before them, i.e.
                                       where the §7 safeguard would replace the fit; counted
                                       whether or not opts.safeguard applies it (extraction
                                       only, not refinement sweeps) */
  EXTERND_STATS_LEN = 16
};

/*
 * Test capture of one iteration of one block of the block path (§2.4), for
 * checking every step of it on identical inputs.  Every pointer is a device
 * buffer and may be NULL (that item is not recorded).  Rows are components:
 * a row of P, Vt, Q or Ut holds one column of the paper's n x b or m x b
 * matrix.  bb is the width of the captured block (b, or k mod b for a
 * trailing partial block).  Only the extraction pass is captured, not
 * refinement sweeps.
 */
typedef struct externd_block_capture {
  int64_t block;       /* block index: components [block * b, block * b + bb) */
  int32_t iteration;   /* ALS iteration whose two half-steps are recorded (0-based) */
  int32_t reserved;
  float* R;            /* m x n: the residual the block is fitted to */
  uint32_t* U_in;      /* bb x ceil(m/16) code words: U entering the iteration */
  float* P;            /* bb x n: U^T R, summed over the contraction's splits */
  float* GinvU;        /* bb x bb: (U^T U + eps I)^-1 as applied */
  float* Vt;           /* bb x n: decorrelated V target (P (U^T U + eps I)^-1)^T */
  uint32_t* V;         /* bb x ceil(n/16): T_tau of each row of Vt */
  float* Q;            /* bb x m: (R diag(w) V)^T (w = 1 unless importance weighted) */
  float* GinvV;        /* bb x bb: (V^T diag(w) V + eps I)^-1 as applied */
  float* Ut;           /* bb x m: decorrelated U target */
  uint32_t* U_out;     /* bb x ceil(m/16): T_tau of each row of Ut */
  double* rhs;         /* bb: u_j . q_j of the final iteration (joint-solve right side) */
} externd_block_capture;

/*
 * Optional knobs of externd_decompose.  Zero-initialise, set struct_size to
 * sizeof(externd_opts), then set what you need.  A NULL opts means defaults.
 */
typedef struct externd_opts {
  uint32_t struct_size;   /* sizeof(externd_opts) */
  uint32_t reserved0;
  uint64_t seed;          /* starting-vector seed (default 0) */
  int32_t mode;           /* enum externd_mode; sequential path only (default AUTO) */
  int32_t reserved1;
  double* trace;          /* device, optional: ||R||^2 after each component
                             (sequential: k entries, predicted from the exact
                             per-step decrease) or after each block (block mode:
                             ceil(k/b) entries) */
  int64_t* stats;         /* device, optional: EXTERND_STATS_LEN counters (overwritten) */
  /* Test capture of one component of the sequential path.  It is enabled
   * when capture_component >= 0 and at least one capture pointer is
   * non-NULL (a zero-initialised opts captures nothing); each pointer may be
   * NULL. */
  int64_t capture_component;
  float* capture_R;       /* m*n: residual before the component (row-resident copy) */
  float* capture_Rcol;    /* m*n: the same residual from the column-resident copy */
  float* capture_R_next;  /* m*n: residual after the component's deflation */
  float* capture_y;       /* iters*n: y_t = R^T u_{t-1} */
  float* capture_x;       /* iters*m: x_t = R v_t */
  int8_t* capture_v;      /* iters*n: v_t */
  int8_t* capture_u;      /* iters*m: u_t (u_0 is the seeded start) */
  float* capture_d;       /* 1: the component's scale */
  /* Caller-owned device workspace (optional).  When non-NULL it must be
   * 256-byte aligned and hold at least externd_workspace_bytes(...) bytes for
   * the same arguments; the library then allocates nothing.  Its contents are
   * scratch: nothing is expected in it and nothing is left for the caller.
   * Two calls in flight at once must not share one workspace. */
  void* workspace;
  uint64_t workspace_bytes;
  double* norm_a2;        /* device, optional: receives ||A||_F^2 (fp64) */
  /* Refinement sweeps (§2.4, block mode only; EXTERND_EINVAL when the block
   * width is 1).  After extraction every sweep revisits the blocks in order:
   * the block is added back to R, its iterations run again from its stored U,
   * the scales are solved jointly, and the refit replaces the block when its
   * predicted decrease of ||R||^2 is at least the stored block's (measured
   * exactly while adding it back), else the stored block is deflated again.
   * The energy therefore never falls from sweep to sweep (up to the fp32
   * rounding of the deflations). */
  int32_t sweeps;         /* default 0 */
  /* Ternarizer (§2.2): EXTERND_TERN_MEAN (default) is T_tau; with
   * EXTERND_TERN_PROJECTION every ternarization is the optimal ternary
   * projection (keep the s largest |x| maximising their sum over sqrt(s);
   * tau is unused).  The projection runs in streaming and block mode only
   * (AUTO picks streaming) and needs m, n <= 16384; otherwise
   * EXTERND_EUNSUPPORTED. */
  int32_t ternarizer;
  double* sweep_trace;    /* device, optional: sweeps entries, predicted ||R||^2 after each sweep */
  /* Importance-weighted ALS (§2.5, every mode).  importance: device, n
   * per-input-channel second moments h >= 0 (e.g. from an importance matrix);
   * the column weights are w_j = h_j / max(h) + importance_lambda, computed
   * in fp32 on the device (w = lambda when h is all zero).  The objective is
   * sum_ij w_j (A - B diag(D) C)_ij^2: the u update targets R diag(w) v, the v
   * update keeps the plain R^T u, d = u^T R diag(w) v / (|u|^2 v^T diag(w) v)
   * (0 when v^T diag(w) v = 0), block mode uses the Gram V^T diag(w) V, and
   * energy, trace, sweep_trace and norm_a2 are the weighted sums.  Negative or
   * non-finite entries of h count as non-finite input (energy NaN). */
  const float* importance;
  float importance_lambda; /* >= 0, finite (default 0) */
  /* Single-entry safeguard (appendix §7, monotone residual decrease): when
   * the fitted component lowers ||R||^2 by less than max_ij w_j R_ij^2 (the
   * decrease of the single entry e_r e_c^T with d = R_rc), replace it by that
   * entry; the smallest row-major index r n + c takes a tie.  0 (default)
   * leaves every fit as it is; stats[EXTERND_STAT_SAFEGUARD] counts the
   * would-be replacements either way.  1 applies it: sequential path only,
   * run in streaming mode (AUTO picks streaming; RESIDENT and block mode give
   * EXTERND_EUNSUPPORTED). */
  int32_t safeguard;
  const externd_block_capture* block_capture; /* HOST pointer, optional (block mode) */
} externd_opts;

/*
 * Decompose A (m x n, fp32, row-major) into k = externd_rank(m, n, mu)
 * components.  §2.3 (block <= 1) or §2.4 (block > 1).
 *   mu     > 0, finite: inner-rank multiplier (§2.1).
 *   tau    >= 0, finite: threshold scale of T_tau (§2.2), used as fp32.
 *   iters  >= 1: alternating-fit iterations per component / block (§2.3: 15).
 *   block  <= 1: sequential greedy ALS; otherwise block ALS with
 *          b = externd_block_width(m, n, block) (falls back to sequential if < 2;
 *          EXTERND_EUNSUPPORTED if b > EXTERND_MAX_BLOCK).
 * Outputs (device): B2 [k][ceil(m/16)] u32, C2 [k][ceil(n/16)] u32, D [k] fp32,
 *   energy [1] fp64 = 1 - ||A - B diag(D) C||^2 / ||A||^2 of the fp32 residual
 *   (1 when ||A|| = 0; NaN when A has non-finite entries).
 * A is not modified.  Workspace is opts->workspace when given (EXTERND_ENOMEM if
 * smaller than externd_workspace_bytes, EXTERND_EINVAL if not 256-byte
 * aligned), else allocated and freed stream-ordered on `stream`.
 */
int externd_decompose(const float* A, int64_t m, int64_t n, float mu, float tau,
                      int32_t iters, int32_t block, void* stream,
                      uint32_t* B2, uint32_t* C2, float* D, double* energy,
                      const externd_opts* opts);

/*
 * externd_decompose for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments and results, on the resident sequential
 * path only (block widths above 1, EXTERND_MODE_STREAMING and shapes that do
 * not fit on chip give EXTERND_EUNSUPPORTED; opts->workspace must be NULL).
 * Its scratch memory is a static 256 KiB device array per GPU, held until
 * the process ends, so it calls no allocator; it holds one placement of the
 * exchange words (16 KB (ceil(m/1024) + ceil(n/1024)) rounded up to 16 KB,
 * plus 2 KB), so this entry point skips the placement probe that
 * externd_decompose runs for long decompositions (the factors are the
 * same).  A shape needing more scratch (the words, 4 n + k / 8 bytes, and
 * about 40 KB: 146.5 KiB at 2560 x 2560 with k = 5120) gives
 * EXTERND_ENOMEM.  All calls on
 * one GPU share that array (each call clears what it needs first): calls
 * that overlap on one GPU, on any streams, race and must not be issued.
 */
int externd_decompose_noalloc(const float* A, int64_t m, int64_t n, float mu, float tau,
                              int32_t iters, int32_t block, void* stream,
                              uint32_t* B2, uint32_t* C2, float* D, double* energy,
                              const externd_opts* opts);

/* energy = 1 - ||A - B diag(D) C||^2 / ||A||^2 accumulated in fp64 from the
 * 2-bit factors (§2.1).  k may be 0 (energy 0, or 1 for A = 0). */
int externd_energy(const float* A, int64_t m, int64_t n, const uint32_t* B2,
                   const uint32_t* C2, const float* D, int64_t k, void* stream,
                   double* energy);

/* A_hat = B diag(D) C (m x n fp32 row-major), accumulated in fp64 per entry (§2.1). */
int externd_reconstruct(const uint32_t* B2, const uint32_t* C2, const float* D,
                        int64_t m, int64_t n, int64_t k, void* stream, float* A_hat);

/* Inference with the factors (§2.6): y = B (diag(D) (C x)) for x of length n,
 * y of length m.  C x and B w are sums of signed copies (no multiplies; k
 * multiplies for w = D * C x), accumulated in fp32 in a fixed order.  B2, C2,
 * D as produced by externd_decompose; k may be 0 (y = 0).  Workspace of about
 * 4 (k + m k / 64) bytes is allocated and freed stream-ordered. */
int externd_apply(const uint32_t* B2, const uint32_t* C2, const float* D, int64_t m, int64_t n,
                  int64_t k, const float* x, void* stream, float* y);

/* Transpose a 2-bit code matrix (the §2.6 storage: 16 codes per uint32, code
 * j of a word in bits 2j, 2j+1): src holds `rows` rows of `cols` codes,
 * ceil(cols/16) words per row; dst receives `cols` rows of `rows` codes,
 * ceil(rows/16) words per row, zero padding.  externd_transpose_codes(B2, k,
 * m, ...) turns the component-major B2 of externd_decompose into B row by
 * row, the form externd_apply_rows reads (once per factorisation).  Device
 * pointers owned by the caller, dst not overlapping src; enqueued on
 * `stream`.  EXTERND_EINVAL for a negative size or a null pointer with
 * nonzero sizes. */
int externd_transpose_codes(const uint32_t* src, int64_t rows, int64_t cols, void* stream, uint32_t* dst);

/* y = B (diag(D) (C x)) (§2.6) with B given row by row: BT2 holds m rows of
 * ceil(k/16) words (externd_transpose_codes of B2); C2 and D as produced by
 * externd_decompose; x has n entries, y receives m.  Both products run on
 * int8 MFMA: the vector (x, then w = D (C x) in fp32) is rounded to fixed
 * point with 30 bits below its largest magnitude and split into four int8
 * digits, every ternary sum is an exact integer, and each output is
 * converted once.  So the result is the exact one for the rounded vector
 * (each entry moved by at most 2^-30 of the vector's largest magnitude),
 * independent of summation order and bit-reproducible.  n, k <= 2^21
 * (EXTERND_EINVAL beyond).  A non-finite entry of x, D or w makes y all
 * NaN.  k may be 0 (y = 0).  workspace: NULL, and a workspace of
 * externd_apply_rows_workspace_bytes(m, n, k) bytes (4 k plus a few KiB) is
 * allocated and freed stream-ordered; or a caller device buffer, 256-byte
 * aligned, of at least that many bytes (workspace_bytes), used instead, so
 * that a loop of calls allocates nothing (EXTERND_EINVAL if too small or
 * misaligned).  Calls that overlap on one workspace race. */
int externd_apply_rows(const uint32_t* BT2, const uint32_t* C2, const float* D, int64_t m, int64_t n,
                       int64_t k, const float* x, void* stream, float* y, void* workspace,
                       size_t workspace_bytes);

/* Workspace bytes externd_apply_rows needs for this shape on the current
 * device; 0 for an invalid shape or device. */
size_t externd_apply_rows_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* k = mu * min(m, n) rounded half away from zero in fp64 (§2.1); -1 on bad input. */
int64_t externd_rank(int64_t m, int64_t n, float mu);

/* Rank needed for a target energy (§3.3: choosing mu per matrix), read off
 * one decomposition's trace thanks to the greedy prefix property: the run at
 * a smaller rank is the prefix of the run at a larger one (in block mode the
 * smaller rank must be a whole number of blocks).  HOST arrays: trace[j] is
 * ||R||^2 after component j (sequential, step = 1) or after block j (block
 * mode, step = b); total is the decomposition's k; norm_a2 its ||A||^2
 * (externd_opts.norm_a2).  Returns the smallest c = min((j+1) step, total)
 * with 1 - trace[j] / norm_a2 >= target, 0 when norm_a2 = 0, -1 when no
 * prefix reaches the target, and -2 on invalid arguments.  mu = c / min(m, n)
 * reproduces c through externd_rank.  energy (HOST, may be NULL) receives the
 * energy of the returned prefix: 1 - trace[j] / norm_a2, 1 when norm_a2 = 0,
 * NaN when no prefix reaches the target or the arguments are invalid. */
int64_t externd_rank_for_energy(const double* trace, int64_t len, int64_t total, int32_t step,
                                double norm_a2, double target, double* energy);

/* Block width of a request: min(block, floor(min(m,n)/8)), 1 meaning
 * sequential (§2.4).  The block kernels take widths up to
 * EXTERND_MAX_BLOCK: externd_decompose returns EXTERND_EUNSUPPORTED for a
 * wider one (e.g. the pages' default 256 on a matrix with min(m, n) >=
 * 2048), rather than silently narrowing the block. */
#define EXTERND_MAX_BLOCK 128
int32_t externd_block_width(int64_t m, int64_t n, int32_t block);

/* 1 if the resident sequential kernel can hold an m x n residual on chip. */
int32_t externd_resident_fits(int64_t m, int64_t n);

/* Bytes of device workspace externd_decompose needs for these arguments
 * (mode as in externd_opts.mode; it only matters for the sequential path).
 * Without opts->workspace the library allocates this much stream-ordered
 * (hipMallocAsync) and frees it stream-ordered before returning.  For the
 * resident path of a long decomposition (k >= 1024 and m n >= 2^20) it
 * includes 8 placements of the exchange words, which a short probe times
 * before the run to keep the fastest (about 852 KB at 2560 x 2560, k =
 * 5120; one placement otherwise).  Returns 0
 * for invalid arguments, or when the AUTO/RESIDENT choice needs the device
 * and no gfx950 device is current; externd_last_error() says which. */
uint64_t externd_workspace_bytes(int64_t m, int64_t n, float mu, int32_t block, int32_t mode);

/* ---- single-step entry points (the same device routines as the streaming path) ---- */

/* codes = T_tau(x) for a length-N fp32 vector (§2.2); nnz (device int32, may
 * be NULL) receives the number of nonzeros. */
int externd_ternarize(const float* x, int64_t N, float tau, void* stream,
                      uint32_t* codes, int32_t* nnz);

/* codes = the optimal ternary projection of a length-N fp32 vector (§2.2):
 * the s largest |x_j| keep their signs, s maximising their sum over sqrt(s);
 * the sort takes equal magnitudes in index order, and prefixes are compared
 * exactly on the fixed-point magnitudes of T_tau's mean.  1 <= N <= 16384
 * (EXTERND_EUNSUPPORTED above).  nnz as for externd_ternarize. */
int externd_project(const float* x, int64_t N, void* stream, uint32_t* codes, int32_t* nnz);

/* y = R^T u for R (m x n) and u given as 2-bit codes of length m (§2.3 step 1). */
int externd_gemv_t(const float* R, int64_t m, int64_t n, const uint32_t* u_codes,
                   void* stream, float* y);

/* x = R v for v given as 2-bit codes of length n (§2.3 step 1). */
int externd_gemv_n(const float* R, int64_t m, int64_t n, const uint32_t* v_codes,
                   void* stream, float* x);

/* R <- R - d u v^T in place, one fp32 rounding per entry (§2.3 step 3). */
int externd_deflate(float* R, int64_t m, int64_t n, const uint32_t* u_codes,
                    const uint32_t* v_codes, float d, void* stream);

/* Status text and the last error message of the calling thread. */
const char* externd_status_string(int status);
const char* externd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXTERND_H */
