/*
 * ccr_oracle.c -- CPU oracle for the ring all-reduce hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * reference that the GPU library is checked against.  Only the test suite,
 * the package smoke check and the benchmark's cpu_baseline leg may load it.
 * It shares no code, header, table or helper with the GPU library.
 *
 * Source: "HOCCL: Offloading Collective Communication from GPU Cores to
 * Accelerate Distributed Training" (Fei et al.).  The paper itself leaves the
 * reduction out of its offload scope (§5 Limitations: AllReduce and
 * ReduceScatter need compute-unit execution and fall outside HOCCL) and never
 * spells out a ring; what is computed here is the textbook ring
 * reduce-scatter followed by ring all-gather, with every hop a separate
 * point-to-point transfer, as the paper's collective scheduler composes
 * collectives from P2P flows (§3.4 Collective Scheduler, Fig. 6).  The
 * readings taken where the paper is silent are:
 *
 *   R1  rank q sends to rank (q+1) mod R; after reduce-scatter rank c owns
 *       the fully reduced chunk c;
 *   R2  chunk c has Lc = align_up(ceil(N/R), V) elements, V = 16 bytes / elem
 *       size, chunk c = [min(N, c*Lc), min(N, (c+1)*Lc)); each chunk is cut
 *       into S slices the same way (Ls = align_up(ceil(len/S), V));
 *   R3  reduce-scatter step k (k = 0..R-2): every rank q does
 *         b[q][chunk c] = b[q][chunk c] + b[q-1][chunk c],  c = (q-k-2) mod R;
 *       all-gather step k: b[q][chunk c] = b[q-1][chunk c], c = (q-k-1) mod R;
 *   R4  bf16 with fp32 accumulation, "per hop": each hop computes
 *       bf16_rne(float(a) + float(b));  the "fp32 partials" variant carries
 *       the running partial in fp32 and rounds to bf16 once, at the last hop;
 *   R5  rounding is IEEE round-to-nearest-even, no flush of denormals.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off (no fast-math).
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1

/* ------------------------------------------------------------------------ */
/* Partition (reading R2).                                                   */
/* ------------------------------------------------------------------------ */

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t align_up(int64_t a, int64_t v) { return ceil_div(a, v) * v; }
static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
static int mod(int a, int m) { int r = a % m; return r < 0 ? r + m : r; }

/* Bounds of chunk c of a buffer of n elements split over R ranks. */
void orc_chunk_bounds(int64_t n, int R, int vec, int c, int64_t *lo, int64_t *hi)
{
    int64_t len = align_up(ceil_div(n, R), vec);
    *lo = min64(n, (int64_t)c * len);
    *hi = min64(n, (int64_t)(c + 1) * len);
}

/* Bounds of slice s of the element range [clo, chi). */
void orc_slice_bounds(int64_t clo, int64_t chi, int S, int vec, int s,
                      int64_t *lo, int64_t *hi)
{
    int64_t len = chi - clo;
    int64_t sl = align_up(ceil_div(len, S), vec);
    *lo = clo + min64(len, (int64_t)s * sl);
    *hi = clo + min64(len, (int64_t)(s + 1) * sl);
}

/* Element range touched by slice s of chunk c, restricted to the window
 * [wlo, whi) of element indices (the whole buffer, [0, n), except in the
 * range entry point below: every element's operations depend on no other
 * element, so a window sees exactly the operations of the full run). */
static void piece(int64_t n, int R, int S, int vec, int c, int s,
                  int64_t wlo, int64_t whi, int64_t *lo, int64_t *hi)
{
    int64_t clo, chi;
    orc_chunk_bounds(n, R, vec, c, &clo, &chi);
    orc_slice_bounds(clo, chi, S, vec, s, lo, hi);
    if (*lo < wlo) *lo = wlo;
    if (*hi > whi) *hi = whi;
}

/* ------------------------------------------------------------------------ */
/* bfloat16 (reading R4/R5).  bf16 is the top half of an IEEE binary32.      */
/* ------------------------------------------------------------------------ */

float orc_bf16_to_f32(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* Round an fp32 value to the nearest bf16, ties to even.  A NaN maps to a
 * quiet NaN with the same sign. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    if ((bits & 0x7f800000u) == 0x7f800000u && (bits & 0x007fffffu) != 0)
        return (uint16_t)((bits >> 16) | 0x0040u);
    uint32_t lsb = (bits >> 16) & 1u;
    return (uint16_t)((bits + 0x7fffu + lsb) >> 16);
}

void orc_f32_to_bf16_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_bf16(in[i]);
}

void orc_bf16_to_f32_array(const uint16_t *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_bf16_to_f32(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Ring reduce-scatter and all-gather, simulated hop by hop (reading R3).    */
/* Work is slice-major: all steps of slice 0, then slice 1, ...  Values do   */
/* not depend on S; S only changes which elements a hop moves at a time.     */
/* ------------------------------------------------------------------------ */

static void rs_step_f32(float *const *b, int R, int64_t n, int S, int s, int k,
                        int64_t wlo, int64_t whi)
{
    for (int q = 0; q < R; q++) {
        int c = mod(q - k - 2, R), p = mod(q - 1, R);
        int64_t lo, hi;
        piece(n, R, S, 4, c, s, wlo, whi, &lo, &hi);
        for (int64_t i = lo; i < hi; i++) b[q][i] = b[q][i] + b[p][i];
    }
}

static void ag_step(void *const *b, int R, int64_t n, int S, int s, int k,
                    int esize, int64_t wlo, int64_t whi)
{
    int vec = 16 / esize;
    for (int q = 0; q < R; q++) {
        int c = mod(q - k - 1, R), p = mod(q - 1, R);
        int64_t lo, hi;
        piece(n, R, S, vec, c, s, wlo, whi, &lo, &hi);
        if (hi > lo)
            memcpy((char *)b[q] + lo * esize, (char *)b[p] + lo * esize,
                   (size_t)(hi - lo) * esize);
    }
}

static void rs_step_bf16(uint16_t *const *b, int R, int64_t n, int S, int s, int k,
                         int64_t wlo, int64_t whi)
{
    for (int q = 0; q < R; q++) {
        int c = mod(q - k - 2, R), p = mod(q - 1, R);
        int64_t lo, hi;
        piece(n, R, S, 8, c, s, wlo, whi, &lo, &hi);
        for (int64_t i = lo; i < hi; i++)
            b[q][i] = orc_f32_to_bf16(orc_bf16_to_f32(b[q][i]) +
                                      orc_bf16_to_f32(b[p][i]));
    }
}

/* fp32-partials variant: part[q] is rank q's fp32 partial for the chunk it
 * last reduced; the value that travels from q-1 to q at step k>0 is
 * part[q-1], at step 0 it is the bf16 input of q-1.  The last hop rounds. */
static void rs_step_bf16_p32(uint16_t *const *b, float *const *part, int R,
                             int64_t n, int S, int s, int k, int64_t wlo, int64_t whi)
{
    for (int q = 0; q < R; q++) {
        int c = mod(q - k - 2, R), p = mod(q - 1, R);
        int64_t lo, hi;
        piece(n, R, S, 8, c, s, wlo, whi, &lo, &hi);
        for (int64_t i = lo; i < hi; i++) {
            float in = (k == 0) ? orc_bf16_to_f32(b[p][i]) : part[p][i];
            float acc = in + orc_bf16_to_f32(b[q][i]);
            if (k == R - 2) b[q][i] = orc_f32_to_bf16(acc);
            else part[q][i] = acc;
        }
    }
}

/* dtype: 0 = fp32, 1 = bf16 per-hop, 2 = bf16 with fp32 partials.
 * part: R scratch fp32 buffers of n elements, only used by dtype 2. */
int orc_ring_reduce_scatter(void *const *b, float *const *part, int R,
                            int64_t n, int S, int dtype)
{
    if (R < 1 || S < 1 || n < 0 || dtype < 0 || dtype > 2) return ORC_EINVAL;
    if (dtype == 2 && R > 1 && part == NULL) return ORC_EINVAL;
    for (int s = 0; s < S; s++)
        for (int k = 0; k + 1 < R; k++) {
            if (dtype == 0) rs_step_f32((float *const *)b, R, n, S, s, k, 0, n);
            else if (dtype == 1) rs_step_bf16((uint16_t *const *)b, R, n, S, s, k, 0, n);
            else rs_step_bf16_p32((uint16_t *const *)b, part, R, n, S, s, k, 0, n);
        }
    return ORC_OK;
}

int orc_ring_all_gather(void *const *b, int R, int64_t n, int S, int esize)
{
    if (R < 1 || S < 1 || n < 0 || (esize != 2 && esize != 4)) return ORC_EINVAL;
    for (int s = 0; s < S; s++)
        for (int k = 0; k + 1 < R; k++) ag_step(b, R, n, S, s, k, esize, 0, n);
    return ORC_OK;
}

/* One hop of the ring: phase 0 = reduce-scatter step k, 1 = all-gather step
 * k, both on slice s only. */
int orc_ring_step(void *const *b, float *const *part, int R, int64_t n, int S,
                  int s, int k, int phase, int dtype)
{
    if (R < 1 || S < 1 || n < 0 || dtype < 0 || dtype > 2) return ORC_EINVAL;
    if (s < 0 || s >= S || k < 0 || k > R - 2 || phase < 0 || phase > 1) return ORC_EINVAL;
    if (phase == 1) {
        ag_step(b, R, n, S, s, k, dtype == 0 ? 4 : 2, 0, n);
    } else if (dtype == 0) {
        rs_step_f32((float *const *)b, R, n, S, s, k, 0, n);
    } else if (dtype == 1) {
        rs_step_bf16((uint16_t *const *)b, R, n, S, s, k, 0, n);
    } else {
        if (part == NULL) return ORC_EINVAL;
        rs_step_bf16_p32((uint16_t *const *)b, part, R, n, S, s, k, 0, n);
    }
    return ORC_OK;
}

/* All-reduce = reduce-scatter then all-gather, slice-major: slice s runs all
 * of its reduce-scatter hops, then all of its all-gather hops. */
int orc_ring_allreduce(void *const *b, float *const *part, int R, int64_t n,
                       int S, int dtype)
{
    if (R < 1 || S < 1 || n < 0 || dtype < 0 || dtype > 2) return ORC_EINVAL;
    if (dtype == 2 && R > 1 && part == NULL) return ORC_EINVAL;
    int esize = dtype == 0 ? 4 : 2;
    for (int s = 0; s < S; s++) {
        for (int k = 0; k + 1 < R; k++) {
            if (dtype == 0) rs_step_f32((float *const *)b, R, n, S, s, k, 0, n);
            else if (dtype == 1) rs_step_bf16((uint16_t *const *)b, R, n, S, s, k, 0, n);
            else rs_step_bf16_p32((uint16_t *const *)b, part, R, n, S, s, k, 0, n);
        }
        for (int k = 0; k + 1 < R; k++) ag_step(b, R, n, S, s, k, esize, 0, n);
    }
    return ORC_OK;
}

/* The same all-reduce on the elements of the window [wlo, whi) only: every
 * hop, in the same order, restricted to those indices.  Each element's
 * result depends only on that element of every rank, so running disjoint
 * windows that cover [0, n) -- one after the other or on separate threads --
 * leaves the buffers exactly as orc_ring_allreduce does. */
int orc_ring_allreduce_range(void *const *b, float *const *part, int R, int64_t n,
                             int S, int dtype, int64_t wlo, int64_t whi)
{
    if (R < 1 || S < 1 || n < 0 || dtype < 0 || dtype > 2) return ORC_EINVAL;
    if (dtype == 2 && R > 1 && part == NULL) return ORC_EINVAL;
    if (wlo < 0 || whi > n || wlo > whi) return ORC_EINVAL;
    int esize = dtype == 0 ? 4 : 2;
    for (int s = 0; s < S; s++) {
        for (int k = 0; k + 1 < R; k++) {
            if (dtype == 0) rs_step_f32((float *const *)b, R, n, S, s, k, wlo, whi);
            else if (dtype == 1) rs_step_bf16((uint16_t *const *)b, R, n, S, s, k, wlo, whi);
            else rs_step_bf16_p32((uint16_t *const *)b, part, R, n, S, s, k, wlo, whi);
        }
        for (int k = 0; k + 1 < R; k++) ag_step(b, R, n, S, s, k, esize, wlo, whi);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Closed form of the ring result: element i of chunk c is the left fold     */
/*   ((x[c+1] + x[c+2]) + ... + x[c+R-1]) + x[c]     (ranks mod R)           */
/* i.e. the order in which the partial travels round the ring.               */
/* ------------------------------------------------------------------------ */

int orc_fold(const void *const *x, int R, int64_t n, int dtype, void *out)
{
    if (R < 1 || n < 0 || dtype < 0 || dtype > 2) return ORC_EINVAL;
    int vec = dtype == 0 ? 4 : 8;
    for (int c = 0; c < R; c++) {
        int64_t lo, hi;
        orc_chunk_bounds(n, R, vec, c, &lo, &hi);
        for (int64_t i = lo; i < hi; i++) {
            if (dtype == 0) {
                float acc = ((const float *)x[mod(c + 1, R)])[i];
                for (int j = 2; j <= R; j++) acc = acc + ((const float *)x[mod(c + j, R)])[i];
                ((float *)out)[i] = acc;
            } else if (dtype == 1) {
                uint16_t acc = ((const uint16_t *)x[mod(c + 1, R)])[i];
                for (int j = 2; j <= R; j++)
                    acc = orc_f32_to_bf16(orc_bf16_to_f32(acc) +
                                          orc_bf16_to_f32(((const uint16_t *)x[mod(c + j, R)])[i]));
                ((uint16_t *)out)[i] = acc;
            } else {
                float acc = orc_bf16_to_f32(((const uint16_t *)x[mod(c + 1, R)])[i]);
                for (int j = 2; j <= R; j++)
                    acc = acc + orc_bf16_to_f32(((const uint16_t *)x[mod(c + j, R)])[i]);
                ((uint16_t *)out)[i] = R == 1 ? ((const uint16_t *)x[0])[i]
                                              : orc_f32_to_bf16(acc);
            }
        }
    }
    return ORC_OK;
}

/* Fold at chosen element positions only (for spot checks of large runs). */
int orc_fold_at(const void *const *x, int R, int64_t n, int dtype,
                const int64_t *idx, int64_t m, void *out)
{
    if (R < 1 || n < 0 || dtype < 0 || dtype > 2) return ORC_EINVAL;
    int vec = dtype == 0 ? 4 : 8;
    int64_t len = align_up(ceil_div(n, R), vec);
    for (int64_t t = 0; t < m; t++) {
        int64_t i = idx[t];
        if (i < 0 || i >= n) return ORC_EINVAL;
        int c = (int)(i / len);
        if (dtype == 0) {
            float acc = ((const float *)x[mod(c + 1, R)])[i];
            for (int j = 2; j <= R; j++) acc = acc + ((const float *)x[mod(c + j, R)])[i];
            ((float *)out)[t] = acc;
        } else if (dtype == 1) {
            uint16_t acc = ((const uint16_t *)x[mod(c + 1, R)])[i];
            for (int j = 2; j <= R; j++)
                acc = orc_f32_to_bf16(orc_bf16_to_f32(acc) +
                                      orc_bf16_to_f32(((const uint16_t *)x[mod(c + j, R)])[i]));
            ((uint16_t *)out)[t] = acc;
        } else {
            float acc = orc_bf16_to_f32(((const uint16_t *)x[mod(c + 1, R)])[i]);
            for (int j = 2; j <= R; j++)
                acc = acc + orc_bf16_to_f32(((const uint16_t *)x[mod(c + j, R)])[i]);
            ((uint16_t *)out)[t] = R == 1 ? ((const uint16_t *)x[0])[i] : orc_f32_to_bf16(acc);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Point-to-point transfer through a pool of staging slots (HOCCL §3.3.1,   */
/* DMA-RNIC chunk pipelining; slot states from §3.2 / Fig. 4).  The data    */
/* result is dst == src; the oracle also replays the slot state machine and */
/* reports each transition so that a schedule can be checked against it.    */
/*   states: 0 idle, 1 filling (copy in), 2 draining (copy out)             */
/* A chunk i always uses slot i mod nslots.                                 */
/* ------------------------------------------------------------------------ */

/* events: up to 3*nchunks records of (chunk, slot, new_state).  Returns the
 * number of records, or -1 on an illegal transition. */
int64_t orc_staged_copy(const void *const *src, void *const *dst, int ntransfers,
                        int64_t nbytes, int64_t chunk_bytes, int nslots,
                        void *slot_mem, int32_t *events, int64_t max_events)
{
    if (ntransfers < 0 || nbytes < 0 || chunk_bytes <= 0 || nslots < 1) return -1;
    int *state = (int *)calloc((size_t)nslots, sizeof(int));
    if (!state) return -1;
    int64_t nev = 0, chunk = 0;
#define EMIT(ch, sl, st)                                                     \
    do {                                                                     \
        if (events) {                                                        \
            if (nev >= max_events) { free(state); return -1; }               \
            events[3 * nev] = (int32_t)(ch); events[3 * nev + 1] = (sl);     \
            events[3 * nev + 2] = (st);                                      \
        }                                                                    \
        nev++;                                                               \
    } while (0)
    for (int m = 0; m < ntransfers; m++) {
        for (int64_t off = 0; off < nbytes; off += chunk_bytes, chunk++) {
            int64_t len = min64(chunk_bytes, nbytes - off);
            int sl = (int)(chunk % nslots);
            char *slot = (char *)slot_mem + (int64_t)sl * chunk_bytes;
            if (state[sl] != 0) { free(state); return -1; }
            state[sl] = 1; EMIT(chunk, sl, 1);
            memcpy(slot, (const char *)src[m] + off, (size_t)len);
            if (state[sl] != 1) { free(state); return -1; }
            state[sl] = 2; EMIT(chunk, sl, 2);
            memcpy((char *)dst[m] + off, slot, (size_t)len);
            state[sl] = 0; EMIT(chunk, sl, 0);
        }
    }
#undef EMIT
    free(state);
    return nev;
}

/* ------------------------------------------------------------------------ */
/* All-to-all of variable-size row segments.  counts[r*R + d] rows go from   */
/* rank r to rank d.  On the sender the segments are laid out by            */
/* destination, on the receiver by source, each contiguous.                 */
/* ------------------------------------------------------------------------ */

int orc_alltoall(const void *const *send, void *const *recv, int R,
                 const int64_t *counts, int64_t row_bytes)
{
    if (R < 1 || row_bytes < 0) return ORC_EINVAL;
    for (int r = 0; r < R; r++) {
        int64_t soff = 0;
        for (int d = 0; d < R; d++) {
            int64_t roff = 0;
            for (int rr = 0; rr < r; rr++) roff += counts[rr * R + d];
            int64_t c = counts[r * R + d];
            if (c < 0) return ORC_EINVAL;
            if (c > 0)
                memcpy((char *)recv[d] + roff * row_bytes,
                       (const char *)send[r] + soff * row_bytes,
                       (size_t)(c * row_bytes));
            soff += c;
        }
    }
    return ORC_OK;
}

/* dst row i = src row idx[i]. */
int orc_permute_rows(void *dst, const void *src, const int32_t *idx,
                     int64_t nrows, int64_t nsrc, int64_t row_bytes)
{
    for (int64_t i = 0; i < nrows; i++) {
        if (idx[i] < 0 || idx[i] >= nsrc) return ORC_EINVAL;
        memcpy((char *)dst + i * row_bytes, (const char *)src + (int64_t)idx[i] * row_bytes,
               (size_t)row_bytes);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* MoE expert-parallel dispatch / combine over R ranks.                      */
/* Expert e lives on rank e / Eloc as local expert e % Eloc.                */
/* ------------------------------------------------------------------------ */

/* Top-K expert ids per token, by decreasing logit, ties to the lower id.
 * Softmax is monotone, so the top-K of the softmax is the top-K of the
 * logits; no probabilities are needed to route. */
int orc_moe_topk(const float *logits, int64_t T, int E, int K, int32_t *topk)
{
    if (K < 0 || K > E) return ORC_EINVAL;
    char *taken = (char *)malloc((size_t)E);
    if (!taken) return ORC_EINVAL;
    for (int64_t t = 0; t < T; t++) {
        const float *row = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int k = 0; k < K; k++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0 || row[e] > row[best]) best = e;
            }
            taken[best] = 1;
            topk[t * K + k] = best;
        }
    }
    free(taken);
    return ORC_OK;
}

/* Dispatch plan of one source rank.  Pack order is (destination rank,
 * local expert, token).  For every send row j: src_tok[j] = token.  For every
 * (t, k): slot[t*K + k] = the send row that carries it.  cnt[d] = rows to d,
 * ecnt[e] = rows for expert e. */
int orc_moe_plan(const int32_t *topk, int64_t T, int E, int K, int R,
                 int32_t *src_tok, int32_t *slot, int64_t *cnt, int64_t *ecnt)
{
    if (R < 1 || E % R != 0) return ORC_EINVAL;
    int eloc = E / R;
    for (int d = 0; d < R; d++) cnt[d] = 0;
    for (int e = 0; e < E; e++) ecnt[e] = 0;
    int64_t j = 0;
    for (int d = 0; d < R; d++)
        for (int l = 0; l < eloc; l++) {
            int e = d * eloc + l;
            for (int64_t t = 0; t < T; t++)
                for (int k = 0; k < K; k++)
                    if (topk[t * K + k] == e) {
                        src_tok[j] = (int32_t)t;
                        slot[t * K + k] = (int32_t)j;
                        j++;
                        cnt[d]++;
                        ecnt[e]++;
                    }
        }
    return ORC_OK;
}

/* Receive-side unpack order on rank d: (local expert, source rank, token).
 * ecnt holds R*E counts: ecnt[r*E + e] = rows from rank r for expert e.
 * recv_d holds, per source r in order, r's segment for d, itself ordered by
 * (local expert, token).  exp_row[j] = the recv_d row that lands in expert-
 * major row j. */
int orc_moe_unpack_index(const int64_t *ecnt, int R, int E, int d, int32_t *exp_row)
{
    if (R < 1 || E % R != 0) return ORC_EINVAL;
    int eloc = E / R;
    int64_t j = 0;
    for (int l = 0; l < eloc; l++) {
        int e = d * eloc + l;
        for (int r = 0; r < R; r++) {
            /* start of r's segment in recv_d, then of expert e inside it */
            int64_t start = 0;
            for (int rr = 0; rr < r; rr++)
                for (int ll = 0; ll < eloc; ll++) start += ecnt[rr * E + d * eloc + ll];
            for (int ll = 0; ll < l; ll++) start += ecnt[r * E + d * eloc + ll];
            for (int64_t i = 0; i < ecnt[r * E + e]; i++) exp_row[j++] = (int32_t)(start + i);
        }
    }
    return ORC_OK;
}
