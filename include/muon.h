/*
 * muon.h -- C ABI of libmuon: the Muon optimizer step with SignMuon's 1-bit
 * sign and majority-vote tail, on AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [SM] "SignMuon: Otimização Distribuída de Muon com Eficiência de
 *        Comunicação" (gist.science technical summary), section 2
 *        "Metodologia: Sign-Muon" -- "Mecanismo Central", "Fluxo Algorítmico
 *        (Distribuído)" steps 1-4 and "Eficiência de Comunicação".
 *   [MG] "NVIDIA MegatronによるLLM学習高速化へ向けた新世代オプティマイザの高度化",
 *        paragraphs 「分散モード」 (three matrix products per Newton-Schulz
 *        iteration) and 「SYRK と融合された all-reduce」 (symmetric rank-k
 *        products that write the full matrix).
 *
 * Conventions shared by every call
 *   - All matrices are dense, row-major and contiguous.  Dtype codes are
 *     MUON_F32 (IEEE binary32) and MUON_BF16 (bfloat16, the upper 16 bits of
 *     binary32).
 *   - Every tensor argument is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or retains memory.  Between calls it
 *     keeps only per-device facts set once: each device's CU count, the
 *     dynamic LDS limits of its kernels (kernel attributes), the address of
 *     its fixed 4 MiB scratch array (used by muon_momentum_noalloc only),
 *     three streams of its own (used by ns_orthogonalize and dion_step, see
 *     there) and each host thread's fork and join events.  These are set up
 *     under atomics or a lock, so host threads may call concurrently (on
 *     separate streams and buffers).  Scratch memory is passed in as `workspace`, sized by
 *     the matching *_workspace_bytes query.
 *   - Device pointers must be 16-byte aligned (MUON_EALIGN otherwise).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     kernels on it and never synchronise; device faults surface at the
 *     caller's next synchronisation.  Calls on different streams that share
 *     output or workspace buffers race.
 *   - Every call returns a status: MUON_OK (0) or a negative MUON_E* code.
 *     Arguments are validated before anything is enqueued, so on any error
 *     other than MUON_ELAUNCH nothing was launched.  No exception or abort
 *     crosses the ABI.
 */
#ifndef MUON_H_
#define MUON_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum muon_dtype { MUON_F32 = 0, MUON_BF16 = 1 };

enum muon_status {
  MUON_OK = 0,
  MUON_EINVAL = -1,     /* null pointer, negative or inconsistent size      */
  MUON_EDTYPE = -2,     /* unsupported dtype / precision code               */
  MUON_EALIGN = -3,     /* a device pointer is not 16-byte aligned          */
  MUON_EWORKSPACE = -4, /* workspace missing or smaller than the query says */
  MUON_ELAUNCH = -5,    /* the HIP runtime rejected a kernel launch         */
  MUON_ESPLIT = -6,     /* (ns_workspace_status) a split product's second
                           half gave up waiting for the first half's partial
                           tile; that tile of the output was not written     */
  MUON_ESCRATCH = -7    /* (muon_momentum_noalloc) the problem needs more
                           scratch than the library's fixed array holds     */
};

/* Newton-Schulz working dimensions are padded up to a multiple of this. */
#define MUON_NS_PAD 256
/* Largest worker count accepted by the vote calls. */
#define MUON_MAX_VOTERS 1023
/* most workers whose int8 signs can be summed in int8 */
#define MUON_INT8_MAX_VOTERS 127
/* Largest element count (numel) the elementwise calls accept, and 64 times
 * the largest nwords of majority_vote: 2^38, more than any one device's
 * memory holds even at one byte per entry, and small enough that every
 * launch grid stays within its 32-bit limit.  Larger: MUON_EINVAL. */
#define MUON_MAX_NUMEL (INT64_C(1) << 38)

/* Human-readable text of a status code (static storage, never NULL). */
const char* muon_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int muon_version(void);

/* muon_time_next_launch -- measurement aid.  The next kernel that the calling
 * host thread launches through this library records `start_event` as it
 * starts and `stop_event` as it ends (hipEvent_t handles created by the
 * caller, either may be NULL), on the stream of that call, so that
 * hipEventElapsedTime gives the kernel's own duration without the gaps
 * around it; then the request is forgotten.  For a call that launches
 * several kernels only the first is timed.  Always MUON_OK. */
int muon_time_next_launch(void* start_event, void* stop_event);

/* ---------------------------------------------------------------------------
 * a1 -- momentum EMA and per-matrix squared Frobenius norm.
 *   [SM] "Fluxo Algorítmico" step 1: each worker updates its local momentum.
 *   The pages print no formula; this computes the EMA
 *       M[i] <- round_m( beta * M[i] + alpha * G[i] )
 *   in place over a flat parameter set of `numel` entries, with alpha =
 *   1 - beta for the classical EMA (heavy-ball momentum is beta, alpha = 1).
 *   The sum of the two exact products is rounded once in fp64, then to fp32
 *   and, for bf16 storage, to bf16 (nearest-even each time).
 *   If `sumsq_out` is not NULL it also writes, for every matrix j of the set,
 *       sumsq_out[j] = sum over its entries of (stored new M)^2,
 *   the squared Frobenius norm the normalisation divides by.  Matrix j covers
 *   flat entries [seg_offsets[j], seg_offsets[j+1]).
 *
 *   M          device, numel entries of m_dtype (F32 or BF16), updated in place
 *   G          device, numel entries of g_dtype (F32 or BF16), read only
 *   seg_offsets device int64[nseg+1], 0 = seg_offsets[0] <= ... <= seg_offsets
 *              [nseg] = numel (only read when sumsq_out != NULL)
 *   sumsq_out  device float[nseg], or NULL to skip the norms
 *   workspace  device scratch of muon_momentum_workspace_bytes(numel, nseg)
 *              bytes (only needed when sumsq_out != NULL)
 *   The sums are deterministic: identical inputs give bit-identical results.
 * ------------------------------------------------------------------------- */
size_t muon_momentum_workspace_bytes(int64_t numel, int nseg);
int muon_momentum(void* M, int m_dtype, const void* G, int g_dtype, int64_t numel,
                  const int64_t* seg_offsets, int nseg, float beta, float alpha,
                  float* sumsq_out, void* workspace, size_t ws_bytes, void* stream);

/* muon_momentum_noalloc -- muon_momentum without a workspace argument, for
 *   callers that cannot allocate device memory: code under HIP graph capture,
 *   tight serving or training loops, harnesses that forbid allocation.  It
 *   computes exactly what muon_momentum computes (same kernels, bit-identical
 *   results) and allocates nothing: the norms' partial sums go to a fixed
 *   4 MiB array in the library's device memory, one per device, held from the
 *   device's first call until the process ends (its address is looked up
 *   once per device on that first call).
 *   Limit: muon_momentum_workspace_bytes(numel, nseg) <= 4 MiB, i.e. about
 *   (524287 - nseg) * 4096 entries (2.1e9); larger problems return
 *   MUON_ESCRATCH before anything is launched.  Without sumsq_out the array
 *   is not used and there is no limit beyond MUON_MAX_NUMEL.
 *   Every call on one device shares that device's array (the last call's
 *   values stay in it; each call writes every partial it reads, so nothing
 *   needs clearing): calls that overlap in time on one device -- on two
 *   streams, or from two host threads -- race and must be ordered by the
 *   caller.  Other arguments and errors as muon_momentum. */
int muon_momentum_noalloc(void* M, int m_dtype, const void* G, int g_dtype, int64_t numel,
                          const int64_t* seg_offsets, int nseg, float beta, float alpha,
                          float* sumsq_out, void* stream);

/* ---------------------------------------------------------------------------
 * a2-a5 -- Newton-Schulz orthogonalisation of a list of momentum matrices.
 *   [SM] "Mecanismo Central" item 1 and "Fluxo" step 1: the polar direction U
 *   of the momentum, approximated by the Newton-Schulz iteration.  For every
 *   problem:
 *       X0 = M / ||M||_F                 (zero matrix -> U = 0)
 *       repeat `steps` times:            ([MG] 「分散モード」: three products)
 *           A = X X^T                    (Gram on the short side; symmetric)
 *           B = b A + c A A              (skipped when c == 0: B = b A)
 *           X = a X + B X
 *       U = X
 *   (a, b, c) are free, so cubic (1.5, -0.5, 0) and quintic coefficient sets
 *   share this call.  For a tall matrix (rows > cols) the iteration runs on
 *   X^T, an exact identity; U is always written in the input's orientation.
 *   The Gram and the polynomial products are symmetric rank-k products
 *   ([MG] 「SYRK と融合された all-reduce」): only lower-triangle tiles are
 *   computed and mirrored into the full matrix.
 *
 *   precision  MUON_BF16: bf16 MFMA operands, fp32 accumulation, X, A and B
 *              held in bf16 between products; the outputs X_1 .. X_k of the
 *              first k iterations also keep their bf16 rounding residual,
 *              which the next iteration adds to its a X term (X + residual
 *              holds X to about 16 significant bits): rounding X costs the
 *              most accuracy while the singular values are still small.  k
 *              is ns_residual_iterations(rows, cols, a, b, c, steps, ...).
 *              A problem whose short side is below ns_bf16_min_side() (96)
 *              runs on the fp32 products instead: at such sizes the bf16
 *              rounding of B alone can exceed 2e-2 relative error, and the
 *              products take microseconds either way.
 *              MUON_F32: fp32 throughout.
 *   problem    M (device, rows x cols of m_dtype), U (device, rows x cols of
 *              u_dtype, may alias nothing else), sumsq (device float holding
 *              sum(M^2), e.g. from muon_momentum, or NULL to compute it),
 *              bits (device, 8-byte aligned, or NULL): the packed signs of U
 *              in sign_pack's layout (ceil(rows * cols / 64) words), i.e.
 *              a6 of [SM] "Fluxo" step 2 on this problem's U.  With bf16
 *              precision, steps > 0, ns_bf16_min_side() <= rows <= cols and
 *              cols % 64 == 0 the signs come from the last product's
 *              epilogue and U may be NULL
 *              (then only the signs are written); otherwise U is required and
 *              the signs are packed from it after the iteration.
 *   Problems of equal shape and dtypes whose pointers are evenly spaced are
 *   batched into one launch per stage (a run).  steps == 0 gives U = X0.
 *   Streams: with two or more runs, the runs are shared out (largest first,
 *   onto the lighter side) between `stream` and a second stream, the first of
 *   the three the library creates once per device (default priority, not
 *   synchronising with the null stream).  The second side starts after the
 *   work already enqueued on `stream` (an event recorded there) and `stream`
 *   waits for it before any later work (an event recorded on the second
 *   stream), so to the caller the call behaves like work on `stream` alone.
 *   The events are the calling host thread's own; host threads share the
 *   library's streams.  If a stream or the events cannot be created, every
 *   run goes on `stream`.
 *   workspace  device, at least ns_workspace_bytes(probs, count, precision)
 *              bytes, 16-byte aligned, owned by the caller; its contents on
 *              entry do not matter (the call clears what must start at zero)
 *              and are undefined on return.  Calls that share a workspace must
 *              not overlap in time.  With two streams it holds the split
 *              scratch and run buffers of each side (the first side's sized
 *              for every run).
 *   Work split: with bf16 operands, a Gram whose contraction is at least
 *   8192 long and whose n_p^2 units (n_p = s / 256, times the batch) fit one
 *   round of the device's CUs (at most 256) runs every off-diagonal 256 x 256
 *   tile as two halves of the contraction and every diagonal tile as one unit
 *   computing only its lower half, instead of n_p (n_p + 1) / 2 whole tiles.
 *   The half that finishes first leaves its fp32 partial tile in the
 *   workspace; the other adds it (two terms: the sum does not depend on
 *   which half came first).  The polynomial product B = bA + cA^2 (which
 *   needs no workspace) runs, when its n_p^2 units per matrix fit one round
 *   of the CUs, as the two 256 x 128 column halves of every off-diagonal tile
 *   plus the lower half of every diagonal tile.  A symmetric product on
 *   256 x 256 tiles that neither splits nor fits one round runs its
 *   off-diagonal tiles whole and its diagonal tiles as lower halves (same
 *   results: every element's contraction order is unchanged).  Results
 *   therefore depend on the device's CU count only through these choices,
 *   and are deterministic on one device.  The second half's wait for the first is bounded
 *   (muon_set_split_wait_limit); a wait that runs out leaves its tile
 *   unwritten and sets an error word in the workspace, which
 *   ns_workspace_status reports.
 * ------------------------------------------------------------------------- */
typedef struct muon_ns_problem {
  const void* M;
  void* U;
  const float* sumsq;
  int64_t rows;
  int64_t cols;
  int32_t m_dtype;
  int32_t u_dtype;
  uint64_t* bits;
} muon_ns_problem;

size_t ns_workspace_bytes(const muon_ns_problem* probs, int count, int precision);
int ns_orthogonalize(const muon_ns_problem* probs, int count, float a, float b, float c,
                     int steps, int precision, void* workspace, size_t ws_bytes,
                     void* stream);

/* ns_residual_iterations -- the k above: how many leading iterations of
 *   ns_orthogonalize keep the bf16 residual of their output, for a rows x cols
 *   problem with these coefficients and steps.  With the residual, the
 *   rounding error of X reaches the next iterate through the slope of B X
 *   alone, p'(x) - a, instead of the slope p'(x) of the scalar map
 *   p(x) = a x + b x^3 + c x^5, which pays while p'(x) >= a / 2.  k is the
 *   larger of steps - 2 (directions far below the typical singular value of
 *   an ill-conditioned momentum keep growing for most iterations) and the
 *   number of iterates p(x0), p(p(x0)), ... of x0 = 1/sqrt(min(rows, cols))
 *   (the typical normalised singular value of a well-conditioned matrix) that
 *   stay below the first x > 0 with p'(x) <= a / 2; at most steps - 1.
 *   Quintic (3.4445, -4.7750, 2.0315), 5 steps: 3; cubic (1.5, -0.5, 0): 4.
 *   Returns k >= 0 (0 for MUON_F32, for a short side below
 *   ns_bf16_min_side(), or a <= 0), or MUON_EINVAL / MUON_EDTYPE. */
int ns_residual_iterations(int64_t rows, int64_t cols, float a, float b, float c, int steps,
                           int precision);

/* ns_bf16_min_side -- the shortest short side that ns_orthogonalize runs on
 *   bf16 products when asked for MUON_BF16 (96); smaller problems run on the
 *   fp32 products (see precision above).  No arguments, no errors. */
int ns_bf16_min_side(void);

/* ns_workspace_status -- did a split product give up?
 *   Enqueues a copy of the workspace's error word to the host on `stream`,
 *   synchronises `stream`, and returns MUON_ESPLIT if a split product that
 *   used this workspace gave up waiting for its other half since the word
 *   was last cleared, else MUON_OK.  ns_orthogonalize clears the word (and
 *   the arrival counters) at the start of every call, so after it the status
 *   describes that call; a stage-call workspace keeps the word until the
 *   caller zeroes its first 1024 bytes again, which it must do after
 *   MUON_ESPLIT (an abandoned tile leaves its counter set).
 *   workspace  device, a workspace of ns_orthogonalize or of the stage calls
 *              (at least 1024 bytes, else MUON_EINVAL; 16-byte aligned).
 *   Copy or synchronisation failures return MUON_ELAUNCH.
 *
 * muon_set_split_wait_limit / muon_get_split_wait_limit -- the number of
 *   polls (each about 128 cycles) a split product's second half makes for
 *   its partner before it gives up; process-wide, read at each launch.
 *   Default 2^22 (seconds: far beyond the microseconds the partner needs,
 *   which depends on no other workgroup).  polls >= 0, else MUON_EINVAL.
 *   0 makes every split second half give up at once: a way to exercise the
 *   error path with every kernel still exiting normally. */
int ns_workspace_status(const void* workspace, size_t ws_bytes, void* stream);
int muon_set_split_wait_limit(int polls);
int muon_get_split_wait_limit(void);

/* Stage calls of the iteration, on padded short-side working buffers.
 * s and l are the padded short and long sides (multiples of MUON_NS_PAD);
 * X is [batch][s][l], A and B are [batch][s][s]; element type is bf16 for
 * MUON_BF16 and fp32 for MUON_F32.  Padding rows/columns must be zero, and
 * stay zero through every stage.
 *
 * ns_normalize (a2): X0[b] = pad(orient(M[b])) * (1/sqrt(sumsq[b])), with the
 *   M matrices rows x cols contiguous one after another, orient = transpose
 *   when rows > cols, and sumsq[b] == 0 giving X0[b] = 0.
 * ns_gram      (a3): A[b] = X[b] X[b]^T.
 * ns_poly      (a4): B[b] = b A[b] + c A[b] A[b]   (A symmetric).
 * ns_apply     (a5): Xout[b] = a X[b] + alpha B[b] X[b]  (X is not read as an
 *   addend when a == 0).  bf16 residuals (MUON_BF16 only, else MUON_EDTYPE;
 *   each may be NULL): with X_lo ([batch][s][l] bf16) the addend is
 *   a (X + X_lo); Xout_lo receives bf16(v - bf16(v)) for each stored value
 *   v of Xout, so that Xout + Xout_lo holds v to about 16 significant bits.
 *   X_lo and Xout_lo may be the same buffer (each entry is read before it is
 *   rewritten, by the same lane); neither may alias X or Xout.
 * One iteration is ns_gram, ns_poly(b, c), ns_apply(a, alpha = 1), or with
 * c == 0 ns_gram, ns_apply(a, alpha = b).
 *
 * sumsq (device float[batch], or NULL; bf16 only, else MUON_EDTYPE) folds the
 * Frobenius scaling into the first iteration: given the raw momentum M as X
 * and sumsq[b] = sum(M[b]^2), ns_gram writes A = M M^T / sumsq and ns_apply
 * writes (a M + alpha B M) / sqrt(sumsq) (0 when sumsq[b] == 0), which is
 * the first iteration on X0 = M / ||M||_F without materialising X0.
 * ns_orthogonalize does this for bf16 momenta that are wide with sides that
 * are multiples of MUON_NS_PAD.
 *
 * workspace (device, or NULL) lets ns_gram split its work as
 * ns_orthogonalize does (see above); with NULL it does not split.  ns_poly
 * and ns_apply take the same workspace (for one call sequence) and currently
 * never split.  It must hold ns_stage_workspace_bytes(s, l, batch, precision)
 * bytes (0 when nothing splits: then it is not used), be 16-byte aligned,
 * and its first 1024 bytes must be zero on the first call: they are arrival
 * counters that every successful call leaves at zero, and the error word of
 * ns_workspace_status.  One workspace sized for
 * (s, l, batch) serves ns_gram(s, l), ns_poly(s) and ns_apply(s, l) on that
 * batch; calls sharing it must not overlap in time.  Too small:
 * MUON_EWORKSPACE. */
int ns_normalize(const void* M, int m_dtype, int64_t rows, int64_t cols, int64_t batch,
                 const float* sumsq, void* X0, int precision, void* stream);
size_t ns_stage_workspace_bytes(int64_t s, int64_t l, int64_t batch, int precision);
int ns_gram(const void* X, void* A, int64_t s, int64_t l, int64_t batch, int precision,
            const float* sumsq, void* workspace, size_t ws_bytes, void* stream);
int ns_poly(const void* A, void* B, int64_t s, int64_t batch, float b, float c,
            int precision, void* workspace, size_t ws_bytes, void* stream);
int ns_apply(const void* B, const void* X, const void* X_lo, void* Xout, void* Xout_lo, int64_t s,
             int64_t l, int64_t batch, float a, float alpha, int precision, const float* sumsq,
             void* workspace, size_t ws_bytes, void* stream);

/* ns_apply_signs (a5 + a6): ns_apply with MUON_BF16 precision (else
 *   MUON_EDTYPE) that also writes the packed signs of Xout, as sign_pack
 *   would pack the stored bf16 values: bits (device, 8-byte aligned) is
 *   [batch][s * l / 64] words, entry b holding Xout[b] (s x l row-major) with
 *   bit i of the flat index in word i >> 6, bit i & 63.  Xout may be NULL:
 *   then only the signs are written (the last iteration of SignMuon needs
 *   nothing else).  X_lo (or NULL) as in ns_apply; no residual is written.
 *   Other arguments, errors and the workspace as ns_apply. */
int ns_apply_signs(const void* B, const void* X, const void* X_lo, void* Xout, uint64_t* bits,
                   int64_t s, int64_t l, int64_t batch, float a, float alpha, int precision,
                   const float* sumsq, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * a6 -- entrywise sign and 1-bit packing.
 *   [SM] "Fluxo" steps 2-3: S = sign(U) in {-1,+1}, packed one bit per entry
 *   for the all-gather exchange ("Eficiência de Comunicação": 32x smaller than
 *   fp32).  Bit i (flat row-major index) is 1 iff !(U[i] < 0), i.e. +1 for
 *   positive, +0.0, -0.0 and NaN.  Layout: word i>>6, bit i&63 (LSB first),
 *   little-endian 64-bit words; the ceil(numel/64)*64 - numel padding bits of
 *   the last word are 0.
 *   U     device, numel entries of u_dtype
 *   bits  device uint64[ceil(numel/64)]
 * ------------------------------------------------------------------------- */
int sign_pack(const void* U, int u_dtype, int64_t numel, uint64_t* bits, void* stream);

/* ---------------------------------------------------------------------------
 * a7 -- majority vote over M packed sign buffers.
 *   [SM] "Mecanismo Central" item 3: S_bar = sign(sum_m S^(m)), an integer sum
 *   of signs and a local threshold.  With sign(0) := +1 this is: out bit = 1
 *   iff 2 * (number of buffers with bit 1) >= M.  Bit-exact.
 *   bits  device uint64[M][nwords] (buffer k at bits + k*nwords)
 *   out   device uint64[nwords]; padding bits follow the same rule (a padding
 *         bit 0 in every buffer votes 0 only when M >= 1: 2*0 >= M is false).
 *   1 <= M <= MUON_MAX_VOTERS.
 * ------------------------------------------------------------------------- */
int majority_vote(const uint64_t* bits, int M, int64_t nwords, uint64_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * a8 -- update W <- W - eta * S_bar.
 *   [SM] "Fluxo" step 4.  Per entry: W[i] <- round_w( fp32(W[i]) - s_i*eta )
 *   with s_i = +1 if vote bit i is 1, else -1; one IEEE fp32 subtraction,
 *   then round-to-nearest-even to bf16 for bf16 storage.  Bit-exact.
 *   W          device, numel entries of w_dtype, updated in place
 *   vote_bits  device uint64[ceil(numel/64)]
 * ------------------------------------------------------------------------- */
int apply_update(void* W, int w_dtype, int64_t numel, const uint64_t* vote_bits, float eta,
                 void* stream);

/* a7 + a8 fused: the vote of M buffers applied straight to W, without
 * writing the vote bits.  Same result as majority_vote then apply_update. */
int vote_and_update(void* W, int w_dtype, int64_t numel, const uint64_t* bits, int M,
                    float eta, void* stream);

/* ---------------------------------------------------------------------------
 * The int8 exchange format ([SM] "Mecanismo Central" item 3; "Fluxo" step 3,
 * the all-reduce variant; "Eficiência de Comunicação": 8 bits per entry,
 * 4x less than fp32).  Each worker's signs travel as int8 +1/-1, an integer
 * SUM all-reduce adds them, and each worker thresholds the sum locally.  On
 * one GPU the M workers' int8 buffers are resident and sum_int8 forms the
 * sum the all-reduce would deliver.  threshold_pack(sum_int8(sign_int8(U_k)))
 * equals majority_vote(sign_pack(U_k)) bit for bit.
 *
 * sign_int8       S[i] = +1 if !(U[i] < 0) (the rule of sign_pack), else -1.
 *                 U device, numel entries of u_dtype; S device int8[numel].
 * sum_int8        out[i] = sum_k S[k*numel + i] for 1 <= M <=
 *                 MUON_INT8_MAX_VOTERS (the sum fits int8; larger M:
 *                 MUON_EINVAL).  S device int8[M][numel]; out device int8[numel].
 * threshold_pack  bit i of bits = 1 iff sum[i] >= 0 (sign(0) := +1), in the
 *                 layout of sign_pack; padding bits 0.  sum device
 *                 int8[numel]; bits device uint64[ceil(numel/64)], ready for
 *                 apply_update.
 * All pointers 16-byte aligned (MUON_EALIGN).  Bit-exact.
 * ------------------------------------------------------------------------- */
int sign_int8(const void* U, int u_dtype, int64_t numel, int8_t* S, void* stream);
int sum_int8(const int8_t* S, int M, int64_t numel, int8_t* out, void* stream);
int threshold_pack(const int8_t* sum, int64_t numel, uint64_t* bits, void* stream);

/* ---------------------------------------------------------------------------
 * Local re-orthogonalisation of the vote ([SM] "Fluxo" step 5, optional: a
 * local polar step on the aggregated sign matrix, with no communication).
 * Per matrix: S_bar (+-1) -> ns_orthogonalize (||S_bar||_F = sqrt(rows*cols))
 * -> W <- W - eta * NS(S_bar):
 *     unpack_signs(vote, ...)  ->  ns_orthogonalize(S_bar -> U)  ->
 *     apply_update_dense(W, U, eta)
 *
 * unpack_signs        out[i] = +1 if bit i of bits is 1, else -1, as
 *                     out_dtype (F32 or BF16; exact).  bits device
 *                     uint64[ceil(numel/64)]; out device, numel entries.
 * apply_update_dense  W[i] <- round_w(fp64(W[i]) - fp64(eta) * fp64(U[i])):
 *                     eta * U is exact in fp64, the difference is rounded
 *                     once to fp32, then (bf16 storage) to bf16.  W device,
 *                     numel of w_dtype, in place; U device, numel of u_dtype.
 *                     Bit-exact.
 * All pointers 16-byte aligned (MUON_EALIGN).
 * ------------------------------------------------------------------------- */
int unpack_signs(const uint64_t* bits, int64_t numel, void* out, int out_dtype, void* stream);
int apply_update_dense(void* W, int w_dtype, int64_t numel, const void* U, int u_dtype, float eta,
                       void* stream);

/* ---------------------------------------------------------------------------
 * Dion (the Dion page's algorithm: low-rank power iteration with error
 * feedback), fp32.  Per matrix X (rows m x cols n) with momentum M, gradient
 * G and previous right factor Q (n x rank, row-major):
 *     B = M + G                      (rounded once to fp32; stored in M)
 *     P = orth(B Q)                  (m x rank; thin QR factor, R diagonal >= 0)
 *     R = B^T P                      (n x rank)
 *     M = B - (1 - mu) P R^T         (error feedback)
 *     Q = ColumnNormalize(R)         (zero columns stay zero)
 *     X = X - eta P Q^T
 * orth: Cholesky-QR applied twice; a column whose residual is at most 1e-4
 * of its own norm counts as dependent and becomes zero, and so does every
 * column after the first min(m, n) independent ones (B Q has rank at most
 * min(m, n); an fp32 Gram cannot resolve a dependent column's residual below
 * about sqrt(2^-24) = 2.4e-4 of its norm, so a rank above a side relies on
 * this bound).  The
 * page does not spell out the orthonormalisation; this is the thin QR factor.
 *
 * problem    M, G, X device fp32 m x n (M, X updated in place, G read);
 *            Q device fp32 n x rank (read as Q_{t-1}, written as Q_t).
 * rank       1 .. MUON_DION_MAX_RANK (the Gram of P is factored in LDS).
 * Problems of equal shape whose M, G, X and Q advance by constant strides
 * (in order of shape and address) run batched.  Pointers 16-byte aligned
 * (MUON_EALIGN).  Limits of the products' launch grids: rows and cols at most
 * 4,194,240 (65535 tiles of 64), count at most 4095, and under 2^32 tiles of
 * 64 x 64 (times 48 for the rank-wide products) per product; beyond them
 * dion_step returns MUON_EINVAL before launching anything and
 * dion_workspace_bytes returns 0.
 * Streams: the runs (one per shape) are shared out, largest first onto the
 * side with the least work, between `stream` and up to three streams of the
 * library's (one side per run, at most four), forked from `stream` with an
 * event and joined back into it, as in ns_orthogonalize: to the caller the
 * call behaves like work on `stream` alone, and every run computes what it
 * computes in a call of its own.
 * workspace  dion_workspace_bytes(probs, count, rank) bytes, 16-byte aligned,
 *            owned by the caller; contents on entry do not matter.  It holds
 *            each run's P and R, the Grams and their inverse factors, a
 *            split-k buffer per side and a 16 KB page of zeros.  Calls that
 *            share a workspace must not overlap in time.
 * ------------------------------------------------------------------------- */
#define MUON_DION_MAX_RANK 192

typedef struct muon_dion_problem {
  void* M;
  const void* G;
  void* X;
  void* Q;
  int64_t rows;
  int64_t cols;
} muon_dion_problem;

size_t dion_workspace_bytes(const muon_dion_problem* probs, int count, int rank);
int dion_step(const muon_dion_problem* probs, int count, int rank, float mu, float eta,
              void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H_ */
