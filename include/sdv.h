/*
 * sdv.h - C ABI of libsdv: the per-step hot path of confidence-scheduled
 * speculative decoding on one MI355X (gfx950) GPU.
 *
 * Three operations, each asynchronous on a caller-given HIP stream:
 *
 *   sd_schedule      survival products, candidate sort and the greedy
 *                    Theta = tau * SPS(B) verify-batch selection
 *   sd_verify        lossless rejection sampling over full vocabulary rows
 *   sd_markov_draft  the low-rank Markov drafting head and the confidence head
 *
 * and around them: sd_rnn_draft (the RNN form of the drafting head), the
 * budget planner (sd_lightspec_update, sd_lightspec_plan) and sd_uniforms
 * (the uniforms behind the random decisions).
 *
 * Sources, by page and section:
 *   [DS]  "DSpark: Confidence-Scheduled Speculative Decoding with
 *         Semi-Autoregressive Generation" (paper summary page):
 *         "innovation one" (parallel backbone + Markov head), "2.1 confidence
 *         head", "2.2 hardware-aware prefix scheduler", Figure 1,
 *         "challenge 2: async scheduling and ZOS compatibility".
 *   [SD]  speculative-decoding history page: "1.1 mechanism" (parallel
 *         verification, rejection sampling, discard after the first
 *         rejection, losslessness); DSpark "move one" (Markov head,
 *         low-rank V x V table), "move two" (survival products), "move three"
 *         (greedy scheduler against a throughput curve).
 *   [LS]  LightSpec article, system section: token slots reserved at the
 *         maximum draft length and cut after the fact (the padded row layout).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *     stated otherwise.  The library never allocates, frees or synchronises;
 *     all scratch lives in a caller-provided workspace of at least
 *     sd_*_workspace_size() bytes (256-byte aligned).  Calls that may run at
 *     the same time (other streams) need workspaces of their own.
 *   - The return value reports host-side argument checks and launch errors
 *     only (SD_OK or a negative SD_E* code).  Nothing is enqueued when an
 *     argument check fails.  Data-dependent faults are reported per request
 *     in a device status array (SD_ST_* bits) with the defined fallbacks
 *     given at each function.
 *   - Random decisions use a counter hash, never device state: SplitMix64
 *     (Steele, Lea, Flood 2014) nested as
 *         h = sm(sm(sm(sm(seed) ^ r) ^ pos) ^ draw),  sm(x) = mix(x + 0x9e3779b97f4a7c15)
 *         u = (h >> 40) * 2^-24
 *     with r the request index, pos = pos0[r] + (1-based draft position) and
 *     draw 0 = draft sample, 1 = accept test, 2 = correction sample.  Calls
 *     are therefore deterministic and replayable for given (seed, pos0).
 *   - Logit rows are row-major with a leading dimension ld (elements, a
 *     multiple of 8 so that every row starts 16-byte aligned); only the first
 *     V entries of a row are read.  V must be a multiple of 8.
 *   - bf16 data is passed as raw 16-bit patterns (uint16_t).
 */
#ifndef SDV_H
#define SDV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDV_ABI_VERSION 4

/* return codes (host side) */
#define SD_OK             0
#define SD_EINVAL        -1   /* bad size, null required pointer, bad mode / dtype / temperature */
#define SD_ERANGE        -2   /* a table or workspace too small for the sizes given */
#define SD_EUNSUPPORTED  -3   /* sizes beyond this build's limits */
#define SD_ELAUNCH       -4   /* the HIP runtime refused a launch */

/* logit dtypes */
#define SD_DTYPE_F32   0
#define SD_DTYPE_BF16  1

/* sd_verify options */
#define SD_VERIFY_STOP_AT_REJECTION 1

/* scheduler modes [DS 2.2, challenge 2] */
#define SD_SCHED_EARLY_STOP     0
#define SD_SCHED_GLOBAL_ARGMAX  1
#define SD_SCHED_CAPPED_TOPK    2
#define SD_SCHED_THRESHOLD      3

/* per-request device status bits */
#define SD_ST_BAD_TOKEN      1   /* token id outside [0, V) */
#define SD_ST_NONFINITE      2   /* a needed logit row holds NaN or +inf */
#define SD_ST_ZERO_Z         4   /* a needed logit row is entirely -inf */
#define SD_ST_ZERO_RESIDUAL  8   /* rejection with no residual mass: drawn from p */
#define SD_ST_ZERO_Q        16   /* q(x) = 0 at a tested draft token */

/* build limits */
#define SD_MAX_GAMMA           255     /* draft positions per request */
#define SD_MAX_SCHED_SLOTS     16384   /* R * gamma_max for sd_schedule */
#define SD_MAX_VOCAB           (1 << 24)

/* ABI version of the loaded library (SDV_ABI_VERSION at build time). */
int sd_abi_version(void);

/* Static text for a return code or for one SD_ST_* bit; never NULL. */
const char* sd_status_string(int code);

/*
 * sd_schedule - hardware-aware prefix scheduler [DS 2.2; SD move two/three].
 *
 * If sts_temp is given, every confidence is first recalibrated by sequential
 * temperature scaling [DS 2.1]: c' = sigmoid(logit(c) / sts_temp[j-1]) for
 * draft position j, computed in fp64 as 1 / (1 + ((1-c)/c)^(1/T)) and rounded
 * to fp32 (c <= 0 gives 0, c >= 1 gives 1, NaN stays NaN).
 * Survival a[r][j] = prod_{i<=j} conf[r][i] (fp32, left to right) is the
 * chance that request r's draft prefix up to position j is accepted.  All
 * candidates (r, j), j = 1..gamma_r[r], are ordered by survival descending,
 * ties by r then j ascending; since a is non-increasing in j every prefix of
 * this order is prefix-closed per request.  tau_n, the expected accepted
 * tokens of the first n candidates, is summed in fixed point
 * (q = rint(a * 2^32), integer prefix sums, tau_n = T_n * 2^-32, exact) and
 *   Theta_n = tau_n * sps[R + n - 1]   (fp64; Theta_0 = 0)
 * where sps[B-1] is the verification throughput at batch B = R + n.
 *   mode EARLY_STOP:    n* = (first n >= 1 with Theta_n < Theta_{n-1}) - 1,
 *                       else N  [DS 2.2: the greedy stop at the first
 *                       drop of the throughput estimate]
 *   mode GLOBAL_ARGMAX: n* = smallest n maximising Theta_n over n = 0..N
 *   mode CAPPED_TOPK:   n* = min(max(*cap_k, 0), N): the capacity was fixed
 *                       before these confidences were known [DS challenge 2];
 *                       pass a previous GLOBAL_ARGMAX call's n_sel pointer as
 *                       cap_k to chain the two without a host round trip.
 *   mode THRESHOLD:     n* = number of candidates with a >= threshold, i.e.
 *                       ell[r] = max{j : a[r][j] >= threshold} [DS
 *                       confidence-threshold sweep]; Theta_{n*} is reported.
 * Then ell[r] = number of selected candidates of request r, batch = R + n*.
 *
 *   R          requests, >= 0;   gamma_max in [0, SD_MAX_GAMMA];
 *              R * gamma_max <= SD_MAX_SCHED_SLOTS
 *   gamma_r    [R] int32 drafted length per request, clamped to
 *              [0, gamma_max]; NULL means gamma_max for all
 *   conf       [R][gamma_max] fp32 confidences in [0, 1] (finite)
 *   sts_temp   [gamma_max] fp32 per-position temperatures (> 0) or NULL
 *   sps        [sps_len] fp32 throughput table, sps[B-1] for batch B;
 *              sps_len >= R * (1 + gamma_max) else SD_ERANGE
 *   cap_k      [1] int32, read in CAPPED_TOPK mode only (device)
 *   threshold  survival threshold, used in THRESHOLD mode only (not NaN)
 *   ell        [R] int32 out
 *   batch, n_sel  [1] int32 out or NULL;  theta [1] fp64 out (Theta_{n*}) or NULL
 *   surv       [R][gamma_max] fp32 out or NULL: a[r][j-1], 0 past gamma_r
 *   workspace  at least sd_schedule_workspace_size(R, gamma_max) bytes,
 *              8-byte aligned (the sorted keys)
 * Two launches (a chip-wide ranking pass, then one workgroup for the scan and
 * the selection); nothing is read back to the host.
 */
size_t sd_schedule_workspace_size(int R, int gamma_max);
int sd_schedule(hipStream_t stream, int R, int gamma_max, const int32_t* gamma_r,
                const float* conf, const float* sts_temp, const float* sps, int sps_len,
                int mode, const int32_t* cap_k, float threshold, int32_t* ell,
                int32_t* batch, int32_t* n_sel,
                double* theta, float* surv, void* workspace, size_t workspace_bytes);

/*
 * sd_verify - lossless verification by rejection sampling [SD 1.1].
 *
 * Request r drafted x_j = draft_tokens[r][j-1], j = 1..ell[r].  Its target
 * row for position j (the row that scores x_j) is tgt_row0[r] + j - 1, for
 * j = 1..ell[r]+1; its draft row for position j is drf_row0[r] + j - 1.
 * (The padded layout of [LS] is tgt_row0[r] = r * (gamma_max + 1),
 * drf_row0[r] = r * gamma_max; a packed layout works as well.)
 * With p_j = softmax(target row / T) and q_j = softmax(draft row / T):
 *   accept x_j iff u(r, pos0[r]+j, 1) * q_j(x_j) < p_j(x_j), i.e. with
 *   probability min(1, p/q); stop at the first rejection j*;
 *   on rejection draw the replacement from max(0, p_j* - q_j*) normalised
 *   (the law that makes the output exactly p, [SD 1.1] losslessness),
 *   otherwise draw a bonus token from p_{ell+1};
 *   draws use the inverse CDF in vocabulary order:
 *   token = min{v : cumsum(w)_v > u * sum(w)} with u = u(r, pos0[r]+pos, 2).
 *
 *   R >= 0; gamma_max in [0, SD_MAX_GAMMA]; V in [8, SD_MAX_VOCAB], V % 8 == 0;
 *   ld >= V, ld % 8 == 0; dtype SD_DTYPE_F32 or SD_DTYPE_BF16; temperature > 0
 *   pos0        [R] int64 or NULL (all 0)
 *   tgt_logits, drf_logits   row-major logit rows (dtype), see above
 *   tgt_row0, drf_row0       [R] int32 first row of each request, >= 0, with
 *                            every row it names inside its buffer (device
 *                            values, not checked)
 *   drf_stats    [R][gamma_max][2] fp32 or NULL: (m, Z) of the draft row of
 *                each position j = 1..gamma_max, in row_stats' format below.
 *                The drafter normalised q_j when it sampled x_j, so it can
 *                hand the normaliser over (sd_markov_draft and sd_rnn_draft
 *                write it as q_stats, at their own temperature, which must be
 *                T).  When given, the draft rows are not streamed: only
 *                q_j(x_j) and the rejected row are read, and the row pass
 *                covers the 1 + ell target rows of each request alone.  A
 *                pair with m = -inf is an all -inf row (ZERO_Z); NaN, m =
 *                +inf, or Z not in (0, inf) marks it NONFINITE.  8-byte
 *                aligned.
 *   draft_tokens [R][gamma_max] int32
 *   ell          [R] int32 verified lengths, clamped to [0, gamma_max]
 *                (typically sd_schedule's output, never read on the host)
 * Outputs:
 *   n_accepted  [R] int32
 *   out_tokens  [R][gamma_max+1] int32: the n_accepted drafts, then the
 *               replacement or bonus token, then -1 padding
 *   status      [R] int32 SD_ST_* bits (written, not OR-ed)
 *   probe_probs [R][gamma_max][2] fp32 (p_j(x_j), q_j(x_j)) for j <= ell, or NULL
 *   row_stats   [R][2*gamma_max+1][2] fp32 (m, Z) with m = max(row)/T and
 *               Z = sum exp(row/T - m): slots 0..gamma_max are target rows of
 *               positions 1..gamma_max+1, slots gamma_max+1.. are draft rows of
 *               positions 1..gamma_max; only slots inside the batch are written
 *               (draft slots copy drf_stats when it is given).  An all -inf
 *               row reports (-inf, 0).  8-byte aligned.
 *   accept_prob [R][gamma_max] fp32 or NULL: alpha_j = sum_v min(p_j(v), q_j(v)),
 *               the probability that position j is accepted given the prefix
 *               was, i.e. 1 - TV(p_j, q_j), the label the confidence head is
 *               trained on [DS 2.1]; 0 past ell and for a failed request.
 *               Costs a second read of every verified row pair (not done
 *               when NULL).
 * options     0 or SD_VERIFY_STOP_AT_REJECTION.  Everything after the first
 *             rejection is discarded [SD 1.1], so the rows past it cannot
 *             change the outcome; with this option each request's rows are
 *             read in rounds of positions (up to 2, 6, 14, ...) and a request
 *             stops being read once it is decided (the request lists and the
 *             recorded draws live in the workspace).  On usable rows the
 *             result is the same; a row past the first rejection is never
 *             read, so it fails nothing (a position fails the request only
 *             when its own target or draft row is unusable, the bonus row
 *             only after full acceptance); row_stats and probe_probs are
 *             written for the rows and positions examined only; accept_prob
 *             must be NULL.  Each round adds two launches: on a batch that
 *             fits the last-level cache (tens of requests at V ~ 150k) the
 *             one-pass call is faster; from ~64 requests at gamma 11 the
 *             rounds are (2x at 256-1024 requests on MI355X).
 * prof_start, prof_stop  optional HIP events (both or neither): recorded on
 *             `stream` right before and after the row-statistics pass (the
 *             bandwidth-bound kernel that streams every row once; its first
 *             round under SD_VERIFY_STOP_AT_REJECTION), so a caller can time
 *             that pass alone.
 * Degenerate data (mirrors the CPU reference): a token outside [0, V) at a
 * tested position sets BAD_TOKEN and counts as a rejection; a needed row with
 * NaN / +inf (NONFINITE) or all -inf (ZERO_Z) fails the request: n_accepted 0
 * and every output token -1 (every batch row is needed, or under
 * SD_VERIFY_STOP_AT_REJECTION the rows up to the first rejection); an empty
 * residual sets ZERO_RESIDUAL and the token is drawn from p_j*; q(x) = 0
 * sets ZERO_Q (accepted iff p(x) > 0).
 */
size_t sd_verify_workspace_size(int R, int gamma_max, int V);
int sd_verify(hipStream_t stream, int R, int gamma_max, int V, int ld, int dtype,
              float temperature, uint64_t seed, const int64_t* pos0,
              const void* tgt_logits, const int32_t* tgt_row0,
              const void* drf_logits, const int32_t* drf_row0, const float* drf_stats,
              const int32_t* draft_tokens, const int32_t* ell,
              int32_t* n_accepted, int32_t* out_tokens, int32_t* status,
              float* probe_probs, float* row_stats, float* accept_prob, int options,
              void* workspace, size_t workspace_bytes,
              hipEvent_t prof_start, hipEvent_t prof_stop);

/*
 * sd_verify_noalloc - sd_verify for callers that cannot allocate device
 * memory: code being captured into a HIP graph, serving loops and harnesses
 * that forbid allocation.  Same arguments, outputs and results as sd_verify,
 * without the workspace (and the timing events): the library holds one
 * workspace of SD_VERIFY_NOALLOC_MAX_WORKSPACE bytes per GPU, a static
 * device array that each GPU the call runs on keeps until the process ends.
 * Sizes whose sd_verify_workspace_size(R, gamma_max, V) exceeds it return
 * SD_ERANGE (R = 256, gamma_max = 11, V = 151936 needs about 3.2 MiB;
 * R = 512, gamma_max = 16 about 8.9 MiB).  No call allocates, frees or
 * clears memory: every workspace word a call reads is written earlier in the
 * same call.  Calls on one GPU share the array, so calls that can overlap
 * (other streams, other threads) race: serialise them on one stream.
 * SD_ELAUNCH if the workspace's device address cannot be obtained.
 */
#define SD_VERIFY_NOALLOC_MAX_WORKSPACE ((size_t)16 << 20)
int sd_verify_noalloc(hipStream_t stream, int R, int gamma_max, int V, int ld, int dtype,
                      float temperature, uint64_t seed, const int64_t* pos0,
                      const void* tgt_logits, const int32_t* tgt_row0,
                      const void* drf_logits, const int32_t* drf_row0, const float* drf_stats,
                      const int32_t* draft_tokens, const int32_t* ell,
                      int32_t* n_accepted, int32_t* out_tokens, int32_t* status,
                      float* probe_probs, float* row_stats, float* accept_prob, int options);

/*
 * sd_markov_draft - semi-autoregressive Markov head plus confidence head
 * [DS innovation one, 2.1; SD move one].
 *
 * For k = 1..gamma, sequentially:
 *   L_k[r]  = bf16_rne( U[r][k-1] + A_k[x_{k-1}] . C_k )     (bias in fp32)
 *   x_k[r]  = inverse-CDF sample of softmax(L_k[r] / T) with u(r, pos0[r]+k, 0)
 *   conf[r][k-1] = sigmoid( w[0:H] . h[r][k-1] + w[H:] . E[x_{k-1}] )
 * starting from the target's anchor x_0 = x0[r] (Figure 1).  B_k(x) =
 * A_k[x] . C_k is the V x V transition table stored low-rank.  L_k is written
 * to q_logits and is exactly the draft distribution that was sampled, so
 * q_logits can be handed to sd_verify as the draft rows (row (r*gamma + k-1),
 * ld = V).
 *
 *   R >= 0; gamma in [0, SD_MAX_GAMMA]; V % 8 == 0, V in [8, SD_MAX_VOCAB];
 *   rank % 32 == 0, 32 <= rank <= 256; H % 8 == 0; rank_e % 8 == 0;
 *   temperature > 0
 *   U        [R][gamma][V] bf16   parallel-backbone logits
 *   A        [gamma][V][rank] bf16   A_k: row x is the left factor of B_k(x)
 *   Ct       [gamma][V][rank] bf16   C_k transposed: row n is column n of C_k
 *   x0       [R] int32 anchors
 *   h        [R][gamma][H] bf16 backbone hidden states
 *   E        [V][rank_e] bf16 Markov embedding;  w [H + rank_e] fp32
 * Outputs: tokens [R][gamma] int32, q_logits [R][gamma][V] bf16,
 *   conf [R][gamma] fp32, status [R] int32, and q_stats [R][gamma][2] fp32
 *   or NULL: (m, Z) of each row L_k[r] with m = max(L_k[r])/T and
 *   Z = sum exp(L_k[r]/T - m) (sd_verify's row_stats format; (-inf, 0) for
 *   an all -inf row), the normaliser the draw used, for sd_verify's
 *   drf_stats.
 * Degenerate data: an anchor outside [0, V) sets BAD_TOKEN and contributes
 * neither bias nor embedding; a row of L_k with NaN / +inf (NONFINITE) or all
 * -inf (ZERO_Z) yields token -1 at that position (and BAD_TOKEN next).
 * Alignment: U, A, Ct, q_logits, h and w 16-byte aligned, q_stats 8-byte
 * aligned, the workspace 256-byte aligned; SD_EINVAL otherwise.
 */
size_t sd_markov_draft_workspace_size(int R, int gamma, int V, int rank);
int sd_markov_draft(hipStream_t stream, int R, int gamma, int V, int rank,
                    float temperature, uint64_t seed, const int64_t* pos0,
                    const uint16_t* U, const uint16_t* A, const uint16_t* Ct,
                    const int32_t* x0, const uint16_t* h, int H,
                    const uint16_t* E, int rank_e, const float* w,
                    int32_t* tokens, uint16_t* q_logits, float* q_stats, float* conf,
                    int32_t* status, void* workspace, size_t workspace_bytes);

/*
 * sd_rnn_draft - the RNN form of the sequential head [DS innovation one]:
 * instead of the previous token alone (Markov head) a recurrent state carries
 * the drafted prefix.  Reading (the page gives no formula): an Elman cell,
 *   s_k = tanh(W s_{k-1} + E_s[x_{k-1}]),  s_0 = 0,  (fp32)
 *   L_k = bf16_rne( U[r][k-1] + s_k . C )     (C shared across positions)
 * with x_k, conf and the degenerate cases exactly as sd_markov_draft (an
 * anchor or token outside [0, V) contributes no embedding term).  The state
 * enters the MFMA product as three bf16 terms (hi = bf16(s), mid = bf16(s -
 * hi), lo = bf16(s - hi - mid)), which carry its fp32 value exactly.
 *   d % 32 == 0, 32 <= d <= 128; other limits as sd_markov_draft
 *   W  [d][d] bf16 (row o: weights of output o);  Es [V][d] bf16
 *   Ct [V][d] bf16: row n is column n of C
 *   U, x0, h, H, E, rank_e, w, outputs as sd_markov_draft
 *   workspace at least sd_rnn_draft_workspace_size(R, gamma, V, d) bytes,
 *   256-byte aligned; W 16-byte aligned, the rest as sd_markov_draft.
 */
size_t sd_rnn_draft_workspace_size(int R, int gamma, int V, int d);
int sd_rnn_draft(hipStream_t stream, int R, int gamma, int V, int d, float temperature,
                 uint64_t seed, const int64_t* pos0, const uint16_t* U, const uint16_t* W,
                 const uint16_t* Es, const uint16_t* Ct, const int32_t* x0, const uint16_t* h,
                 int H, const uint16_t* E, int rank_e, const float* w, int32_t* tokens,
                 uint16_t* q_logits, float* q_stats, float* conf, int32_t* status,
                 void* workspace, size_t workspace_bytes);

/*
 * Training-free two-stage budget planner [LS: two optimisation stages, EMA
 * runtime statistics with interpolation across draft lengths, runtime cost
 * tables].  Readings: the statistics are one EMA per draft position of the
 * acceptance probability alpha_j = sum_v min(p_j, q_j) (sd_verify's
 * accept_prob, [DS 2.1]'s confidence label); the planner feeds them to the
 * prefix scheduler as every request's confidences.
 *
 * sd_lightspec_update - fold one verify step into the table: for position
 * j = 1..gamma_max, over the requests r (in order) with ell[r] >= j whose
 * status has neither NONFINITE nor ZERO_Z, mean_j = (sum alpha[r][j-1]) / n_j
 * in fp64; if count[j-1] == 0 then ema[j-1] = mean_j, else
 * ema[j-1] = (1 - lambda) * ema[j-1] + lambda * mean_j (unfused fp64);
 * count[j-1] += n_j.  Positions with n_j = 0 are left alone.
 *   alpha [R][gamma_max] fp32, ell [R], status [R] int32 (device);
 *   lambda in [0, 1];  ema [gamma_max] fp64 and count [gamma_max] int64 are
 *   caller-owned device state (initialise count to 0 and ema to a prior).
 *
 * sd_lightspec_plan - both stages on the device.
 *   conf_hat[j-1]: ema[j-1] where count > 0; elsewhere linear interpolation
 *     between the nearest positions with count > 0, held constant past the
 *     first / last one; if none has count > 0, ema as given; clamped to [0, 1]
 *     and rounded to fp32.
 *   stage 1 (verify budget): sd_schedule in GLOBAL_ARGMAX mode on
 *     conf[r][j] = conf_hat[j] with gamma_r = d_prev (the previous round's draft
 *     lengths; NULL means gamma_max): ell, batch, n_sel, theta as there.
 *   stage 2 (draft budget): for d = 1..gamma_max with every request drafting
 *     d tokens, n*(d) = smallest n in [0, R d] maximising Theta_n and
 *       phi[d-1] = (R + tau_{n*}) / (draft_cost[d-1] + 1 / sps[R + n* - 1])
 *     (fp64, unfused): expected emitted tokens per unit time when drafting
 *     d tokens costs draft_cost[d-1] and a verify pass at batch B runs
 *     sps[B-1] times per unit time.  d_next = smallest d maximising phi,
 *     b_next = R + n*(d_next).
 *   sps [sps_len] fp32, sps_len >= R * (1 + gamma_max); draft_cost
 *   [gamma_max] fp32; conf_hat [gamma_max] fp32 out or NULL; ell [R], batch,
 *   n_sel, theta as in sd_schedule; d_next, b_next [1] int32 out; phi
 *   [gamma_max] fp64 out or NULL; workspace at least
 *   sd_lightspec_plan_workspace_size(R, gamma_max) bytes, 256-byte aligned.
 *   R * gamma_max <= SD_MAX_SCHED_SLOTS.  Four launches, nothing read back.
 */
int sd_lightspec_update(hipStream_t stream, int R, int gamma_max, const float* alpha,
                        const int32_t* ell, const int32_t* status, double lambda,
                        double* ema, int64_t* count);
size_t sd_lightspec_plan_workspace_size(int R, int gamma_max);
int sd_lightspec_plan(hipStream_t stream, int R, int gamma_max, const double* ema,
                      const int64_t* count, const int32_t* d_prev, const float* sps,
                      int sps_len, const float* draft_cost, float* conf_hat,
                      int32_t* ell, int32_t* batch, int32_t* n_sel, double* theta,
                      int32_t* d_next, int32_t* b_next, double* phi,
                      void* workspace, size_t workspace_bytes);

/*
 * sd_uniforms - the uniforms the library's random decisions draw, for callers
 * that replay or audit a step [SD 1.1: the accept test and the correction
 * sample; DS innovation one: the draft sample]:
 *     out[i] = u(seed, req[i], pos[i], draw)
 * with the counter hash given at the top of this header (req and pos taken
 * as unsigned 64-bit words, so pos[i] = pos0[r] + position reproduces the
 * counter a call with that pos0 used).  The 24-bit values are exact in fp32.
 *   n >= 0; req, pos [n] int64 and out [n] fp32, device memory; draw >= 0
 *   (0 draft sample, 1 accept test, 2 correction sample).
 * Returns SD_EINVAL on a bad size, draw or null pointer (n > 0),
 * SD_EUNSUPPORTED past 2^31 - 1 workgroups, SD_ELAUNCH if the launch fails.
 */
int sd_uniforms(hipStream_t stream, uint64_t seed, long long n, const int64_t* req,
                const int64_t* pos, int draw, float* out);

#ifdef __cplusplus
}
#endif

#endif /* SDV_H */
