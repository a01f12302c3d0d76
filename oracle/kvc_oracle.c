/*
 * kvc_oracle.c -- plain, slow, scalar CPU oracle for softmax-gated token-pool
 * KV compression.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * Sources (the two web pages the method is taken from):
 *   [KP]  vLLM API page "vllm.models.glm5next.amd.ops.kpool_compress"
 *         (Triton kernels _kpool_softmax_rotate_write_cache_kernel,
 *          _kpool_decode_update_batched_kernel and their Python wrappers).
 *   [C128] SGLang page ".../deepseek_v4/c128_online.cuh"
 *         (flash_c128_online_decode, flash_c128_online_prefill,
 *          c128_prefill_forward, plan_online_prefill_host, OnlinePrefillPlan).
 *
 * Precision policy.
 *   - Where the method has a plain mathematical definition the oracle writes
 *     that definition out: the per-channel softmax-weighted mean is evaluated
 *     in double precision (exp from libm), the Walsh-Hadamard rotation as the
 *     exact +-1 matrix product in double.  Values are then rounded to the
 *     storage type the pages use (fp32 accumulator result, bf16 casts).
 *   - Where the pages' fp32 arithmetic decides an integer (the fp8 code via
 *     the fp32 quotient y/scale, the scale via absmax * fp32(1/448)), the
 *     oracle performs that operation in fp32 exactly as the pages do.
 *   - The gated score s = fp32(score) + ape is an fp32 sum on the pages; the
 *     oracle forms it in fp32 too, so the state "max" is bit-reproducible.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-tree-vectorize -fno-fast-math
 *        -shared -fPIC kvc_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Scalar number formats                                                    */
/* ------------------------------------------------------------------------ */

static float u32_as_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_as_u32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one. */
float orc_bf16_to_f32(uint16_t h) { return u32_as_f32((uint32_t)h << 16); }

/* fp32 -> bf16, IEEE round-to-nearest, ties to even.  The pages cast with
 * `.to(tl.bfloat16)` ([KP] softmax kernel, before and after the rotation);
 * that cast rounds to nearest-even.  Definition used here: keep the top 16
 * bits, look at the discarded 16 bits as a fraction of one bf16 ulp; round
 * up when it is above one half, or exactly one half with an odd kept part.
 * Because IEEE patterns are magnitude-ordered, "+1" on the kept part is the
 * next representable magnitude (and carries into the exponent / into inf). */
uint16_t orc_bf16_rne(float f) {
    uint32_t u = f32_as_u32(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)         /* NaN: keep it a quiet NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

float orc_round_bf16(float f) { return orc_bf16_to_f32(orc_bf16_rne(f)); }

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
 * infinities, S.1111.111 is NaN, largest finite 448 = S.1111.110.  The pages
 * name FP8_MAX / FP8_DTYPE without defining them; the target format is OCP
 * e4m3 with max 448. */
double orc_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9)            /* subnormal: m*2^-9 */
                        : ldexp(1.0 + m / 8.0, e - 7);    /* normal          */
    return s ? -v : v;
}

/* fp32 -> e4m3 code, round to nearest, ties to even mantissa.  The pages
 * store an fp32 tensor already clamped to [-448, 448] into an fp8 buffer
 * ([KP] softmax kernel, quantise + store); that cast rounds to nearest-even.
 * Inputs beyond +-448 saturate to +-448 (never reached after the clamp).
 * Signed zero is kept. */
uint8_t orc_e4m3_encode(float q) {
    if (q != q) return 0x7f;
    uint8_t sign = (f32_as_u32(q) >> 31) ? 0x80 : 0x00;
    double a = fabs((double)q);
    if (a >= 448.0) return sign | 0x7e;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: multiples of 2^-9; n == 8 is the smallest normal,
         * whose code (exponent 1, mantissa 0) is also 8. */
        double n = nearbyint(a * 512.0);          /* exact scaling; RNE */
        return sign | (uint8_t)n;
    }
    int E;
    double f = frexp(a, &E);                      /* a = f * 2^E, f in [0.5,1) */
    int e = E - 1;                                /* a = (2f) * 2^e, 2f in [1,2) */
    double n = nearbyint((2.0 * f - 1.0) * 8.0);  /* exact; RNE on 3 bits */
    if (n == 8.0) { n = 0.0; e += 1; }
    int code = ((e + 7) << 3) | (int)n;
    if (code > 0x7e) code = 0x7e;
    return sign | (uint8_t)code;
}

/* Array forms of the scalar conversions (used by the format pins). */
void orc_bf16_rne_array(const float* x, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(x[i]);
}
void orc_e4m3_encode_array(const float* q, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(q[i]);
}

/* ------------------------------------------------------------------------ */
/* Walsh-Hadamard rotation                                                  */
/* ------------------------------------------------------------------------ */

/* y = H x / sqrt(128), H the 128x128 Sylvester-ordered Hadamard matrix,
 * H[i][j] = (-1)^popcount(i & j).  The normalisation is the specification's
 * choice (the rotation helper itself is not printed on [KP]).  The sum of
 * +-x_j for bf16-valued x_j is exact in double; the result is then the
 * correctly rounded fp32 of the exact product. */
void orc_hadamard128(const float* x, float* y) {
    for (int i = 0; i < 128; ++i) {
        double acc = 0.0;
        for (int j = 0; j < 128; ++j) {
            int odd = __builtin_popcount((unsigned)(i & j)) & 1;
            acc += odd ? -(double)x[j] : (double)x[j];
        }
        y[i] = (float)(acc / sqrt(128.0));
    }
}

/* ------------------------------------------------------------------------ */
/* Per-vector scale and quantisation ([KP] softmax kernel, absmax quant)    */
/* ------------------------------------------------------------------------ */

/* Smallest power of two >= t (t > 0, finite).  The pages write
 * exp2(ceil(log2(t))); this is the same number, found from frexp. */
static float pow2_ceil(float t) {
    int E;
    double f = frexp((double)t, &E);              /* t = f * 2^E, f in [0.5,1) */
    if (f == 0.5) return t;                       /* already a power of two */
    return (float)ldexp(1.0, E);
}

/* Quantise a bf16-valued rotated vector y[128]:
 *   a = max(max_d |y_d|, fp32(1e-4));  t = fp32(a * fp32(1/448));
 *   scale = t, or the smallest power of two >= t when round_scale;
 *   code_d = e4m3(clamp(fp32(y_d / scale), -448, 448)). */
static void quantise128(const float* y, int round_scale, uint8_t* code, float* scale_out) {
    float a = 0.0f;
    for (int d = 0; d < 128; ++d) { float v = fabsf(y[d]); if (v > a) a = v; }
    const float floor_ = 1e-4f;
    if (a < floor_) a = floor_;
    const float inv448 = (float)(1.0 / 448.0);
    float t = a * inv448;
    float scale = round_scale ? pow2_ceil(t) : t;
    for (int d = 0; d < 128; ++d) {
        float q = y[d] / scale;
        if (q > 448.0f) q = 448.0f;
        if (q < -448.0f) q = -448.0f;
        code[d] = orc_e4m3_encode(q);
    }
    *scale_out = scale;
}

/* ------------------------------------------------------------------------ */
/* One pool: softmax-gated weighted mean, bf16, rotate, bf16, quantise      */
/* ------------------------------------------------------------------------ */

/* Per channel d over the P slots i of one pool ([KP] softmax kernel, pass 1
 * and pass 2):  s_i = fp32(score_i) + ape_i  (fp32 sum, as on the page),
 *   x_d = sum_i e^{s_i - m} k_i / sum_i e^{s_i - m},  m = max_i s_i,
 * evaluated in double and returned as the fp32 it rounds to.  keys/scores
 * are bf16 patterns; row i of keys starts at keys + i*key_stride. */
void orc_softmax_mean(const uint16_t* keys, int64_t key_stride,
                      const uint16_t* scores, int64_t score_stride,
                      const float* ape, int P, float* x) {
    for (int d = 0; d < 128; ++d) {
        double m = -INFINITY;
        for (int i = 0; i < P; ++i) {
            float s = orc_bf16_to_f32(scores[i * score_stride + d]) + ape[i * 128 + d];
            if ((double)s > m) m = s;
        }
        double num = 0.0, den = 0.0;
        for (int i = 0; i < P; ++i) {
            float s = orc_bf16_to_f32(scores[i * score_stride + d]) + ape[i * 128 + d];
            double p = exp((double)s - m);
            den += p;
            num += p * (double)orc_bf16_to_f32(keys[i * key_stride + d]);
        }
        x[d] = (float)(num / den);
    }
}

/* Full pool-16 epilogue for one pool.  x_out (pre-rounding fp32 mean) and
 * y_out (bf16-valued rotated vector) are optional diagnostics. */
void orc_pool_compress(const uint16_t* keys, int64_t key_stride,
                       const uint16_t* scores, int64_t score_stride,
                       const float* ape, int P, int round_scale,
                       uint8_t* code, float* scale, float* x_out, float* y_out) {
    float x[128], xb[128], h[128], y[128];
    orc_softmax_mean(keys, key_stride, scores, score_stride, ape, P, x);
    for (int d = 0; d < 128; ++d) xb[d] = orc_round_bf16(x[d]);      /* bf16 before rotation */
    orc_hadamard128(xb, h);
    for (int d = 0; d < 128; ++d) y[d] = orc_round_bf16(h[d]);       /* bf16 after rotation  */
    quantise128(y, round_scale, code, scale);
    if (x_out) memcpy(x_out, x, sizeof x);
    if (y_out) memcpy(y_out, y, sizeof y);
}

/* The epilogue alone, from a given fp32 pooled vector x (rows of 128):
 * bf16 round, rotate, bf16 round, quantise.  Used where two fp32 evaluations
 * of the mean legitimately round to different bf16 values. */
void orc_pool_epilogue_rows(const float* x, int64_t rows, int round_scale,
                            uint8_t* code, float* scale) {
    for (int64_t r = 0; r < rows; ++r) {
        float xb[128], h[128], y[128];
        for (int d = 0; d < 128; ++d) xb[d] = orc_round_bf16(x[r * 128 + d]);
        orc_hadamard128(xb, h);
        for (int d = 0; d < 128; ++d) y[d] = orc_round_bf16(h[d]);
        quantise128(y, round_scale, code + r * 128, scale + r);
    }
}

/* Ragged prefill: pool p reads rows pool_src_row[p] .. +P-1 of the packed
 * key / score matrices (row strides in elements).  A NULL pool_src_row means
 * pool p starts at row p*P.  Outputs: code[p*128 + d], scale[p], optional
 * x_dbg[p*128 + d]. */
void orc_compress_prefill(const uint16_t* keys, int64_t key_stride,
                          const uint16_t* scores, int64_t score_stride,
                          const float* ape, const int32_t* pool_src_row,
                          int64_t pool_begin, int64_t pool_end, int P, int round_scale,
                          uint8_t* code, float* scale, float* x_dbg) {
    for (int64_t p = pool_begin; p < pool_end; ++p) {
        int64_t r0 = pool_src_row ? (int64_t)pool_src_row[p] : p * P;
        orc_pool_compress(keys + r0 * key_stride, key_stride,
                          scores + r0 * score_stride, score_stride,
                          ape, P, round_scale, code + p * 128, scale + p,
                          x_dbg ? x_dbg + p * 128 : NULL, NULL);
    }
}

/* Paged output ([KP] softmax kernel, cache-write branch, page size 1): the
 * cache is [num_pages][132] bytes per token page, the 128 e4m3 codes at
 * offset 0 and the fp32 scale at byte offset 128 (the page's scale region
 * starts after page_size*head_dim code bytes).  Pool p goes to page loc[p];
 * pools whose write_mask byte is 0, or whose page is out of range, are not
 * written. */
static void put_paged(uint8_t* cache, int64_t page, const uint8_t* code, float scale) {
    memcpy(cache + page * 132, code, 128);
    memcpy(cache + page * 132 + 128, &scale, 4);
}

void orc_compress_prefill_paged(const uint16_t* keys, int64_t key_stride,
                                const uint16_t* scores, int64_t score_stride,
                                const float* ape, const int32_t* pool_src_row, int64_t n_pools,
                                int P, int round_scale, uint8_t* cache, int64_t num_pages,
                                const int64_t* loc, const uint8_t* write_mask) {
    for (int64_t p = 0; p < n_pools; ++p) {
        if (write_mask && !write_mask[p]) continue;
        int64_t dst = loc[p];
        if (dst < 0 || dst >= num_pages) continue;
        int64_t r0 = pool_src_row ? (int64_t)pool_src_row[p] : p * P;
        uint8_t code[128];
        float scale;
        orc_pool_compress(keys + r0 * key_stride, key_stride, scores + r0 * score_stride,
                          score_stride, ape, P, round_scale, code, &scale, NULL, NULL);
        put_paged(cache, dst, code, scale);
    }
}

/* Pool plan for ragged prefill (the packing the configs describe): sequence
 * b holds seq_lens[b] consecutive rows; its complete pools j are at rows
 * start_b + j*P; tokens after the last complete pool are not compressed.
 * Returns the number of pools, or -1 if cap is exceeded. */
int64_t orc_pool_plan(const int64_t* seq_lens, int64_t batch, int P,
                      int32_t* src_row, int64_t cap) {
    int64_t n = 0, start = 0;
    for (int64_t b = 0; b < batch; ++b) {
        int64_t full = seq_lens[b] / P;
        for (int64_t j = 0; j < full; ++j) {
            if (n >= cap) return -1;
            src_row[n++] = (int32_t)(start + j * P);
        }
        start += seq_lens[b];
    }
    return n;
}

/* ------------------------------------------------------------------------ */
/* Pool-16 decode with a tail ring ([KP] _kpool_decode_update_batched_kernel) */
/* ------------------------------------------------------------------------ */

/* ring: [num_blocks][2][P][128] bf16 (half 0 = key, half 1 = gate score).
 * Request r, token t (in order t = 0..next_n-1), entry e = r*next_n + t:
 *   loc = slot_mapping[e], pos = positions[e], ts = tail_slot_mapping[e]
 *   blk = max(ts, 0) / P
 *   if loc >= 0 && pos >= 0 && pos % P == P-1:  the pool of slots 0..P-1 is
 *       ring slots 0..P-2 plus the current token in slot P-1; compress it and
 *       store (code, scale) at output row loc (rows >= num_out are skipped).
 *   then, if pos >= 0 && ts >= 0: ring[blk][0][pos%P] = key, [1][..] = score.
 * The completion read precedes the stash, and tokens are visited in order, so
 * a completion sees the stashes of earlier tokens of the same request.
 * pool_keys_out / pool_scores_out (nullable, [num_out][P][128]) receive the
 * gathered pool of every completion written to row loc. */
static void ring_decode_impl(uint16_t* ring, int64_t num_blocks, const int32_t* tail_slot_mapping,
                             const uint16_t* key, int64_t key_sb, int64_t key_st,
                             const uint16_t* score, int64_t score_sb, int64_t score_st,
                             const float* ape, const int32_t* slot_mapping,
                             const int32_t* positions, int64_t num_requests, int next_n, int P,
                             int round_scale, uint8_t* out_code, float* out_scale,
                             int64_t num_out, uint16_t* pool_keys_out, uint16_t* pool_scores_out,
                             uint8_t* paged_cache) {
    uint16_t pk[128 * 128], ps[128 * 128];          /* gathered pool, P <= 128 */
    for (int64_t r = 0; r < num_requests; ++r) {
        for (int t = 0; t < next_n; ++t) {
            int64_t e = r * next_n + t;
            int32_t loc = slot_mapping[e], pos = positions[e], ts = tail_slot_mapping[e];
            int64_t blk = (ts > 0 ? ts : 0) / P;
            if (blk >= num_blocks) continue;        /* out-of-range block: nothing */
            uint16_t* ring_k = ring + blk * 2 * P * 128;
            uint16_t* ring_s = ring_k + P * 128;
            const uint16_t* kt = key + r * key_sb + t * key_st;
            const uint16_t* st = score + r * score_sb + t * score_st;
            if (loc >= 0 && pos >= 0 && pos % P == P - 1) {
                for (int i = 0; i < P; ++i) {
                    const uint16_t* srck = (i == P - 1) ? kt : ring_k + i * 128;
                    const uint16_t* srcs = (i == P - 1) ? st : ring_s + i * 128;
                    memcpy(pk + i * 128, srck, 256);
                    memcpy(ps + i * 128, srcs, 256);
                }
                if (loc < num_out && paged_cache) {
                    uint8_t code[128];
                    float scale;
                    orc_pool_compress(pk, 128, ps, 128, ape, P, round_scale, code, &scale,
                                      NULL, NULL);
                    put_paged(paged_cache, loc, code, scale);
                } else if (loc < num_out) {
                    orc_pool_compress(pk, 128, ps, 128, ape, P, round_scale,
                                      out_code + (int64_t)loc * 128, out_scale + loc, NULL, NULL);
                    /* optional copy of the gathered pool, for diagnostics */
                    if (pool_keys_out) memcpy(pool_keys_out + (int64_t)loc * P * 128, pk, P * 256);
                    if (pool_scores_out) memcpy(pool_scores_out + (int64_t)loc * P * 128, ps, P * 256);
                }
            }
            if (pos >= 0 && ts >= 0) {
                int slot = pos % P;
                memcpy(ring_k + slot * 128, kt, 256);
                memcpy(ring_s + slot * 128, st, 256);
            }
        }
    }
}

void orc_ring_decode(uint16_t* ring, int64_t num_blocks, const int32_t* tail_slot_mapping,
                     const uint16_t* key, int64_t key_sb, int64_t key_st,
                     const uint16_t* score, int64_t score_sb, int64_t score_st,
                     const float* ape, const int32_t* slot_mapping, const int32_t* positions,
                     int64_t num_requests, int next_n, int P, int round_scale,
                     uint8_t* out_code, float* out_scale, int64_t num_out,
                     uint16_t* pool_keys_out, uint16_t* pool_scores_out) {
    ring_decode_impl(ring, num_blocks, tail_slot_mapping, key, key_sb, key_st, score, score_sb,
                     score_st, ape, slot_mapping, positions, num_requests, next_n, P, round_scale,
                     out_code, out_scale, num_out, pool_keys_out, pool_scores_out, NULL);
}

/* Ring decode writing completions into a page-size-1 cache (see put_paged);
 * slot_mapping holds the page of each completion. */
void orc_ring_decode_paged(uint16_t* ring, int64_t num_blocks, const int32_t* tail_slot_mapping,
                           const uint16_t* key, int64_t key_sb, int64_t key_st,
                           const uint16_t* score, int64_t score_sb, int64_t score_st,
                           const float* ape, const int32_t* slot_mapping,
                           const int32_t* positions, int64_t num_requests, int next_n, int P,
                           int round_scale, uint8_t* cache, int64_t num_pages) {
    ring_decode_impl(ring, num_blocks, tail_slot_mapping, key, key_sb, key_st, score, score_sb,
                     score_st, ape, slot_mapping, positions, num_requests, next_n, P, round_scale,
                     NULL, NULL, num_pages, NULL, NULL, cache);
}

/* Tail-ring seeding from a prefill batch ([KP] _kpool_tail_seed_kernel).
 * Token i of the batch carries tail slot tslot[i] = block*P + pos%P, or a
 * negative value for padding.  Token i belongs to its request's last P tokens
 * exactly when the token P places ahead is past the batch, is padding, or
 * lies in another block; such a token's key and score rows are copied into
 * slot tslot%P of its block.  Blocks at or beyond num_blocks are skipped. */
void orc_seed_tail_ring(uint16_t* ring, int64_t num_blocks,
                        const uint16_t* key, int64_t key_stride,
                        const uint16_t* score, int64_t score_stride,
                        const int32_t* tslot, int64_t n_tokens, int P) {
    for (int64_t i = 0; i < n_tokens; ++i) {
        int64_t t = tslot[i];
        if (t < 0) continue;
        int64_t blk = t / P;
        int64_t ahead = (i + P < n_tokens) ? (int64_t)tslot[i + P] : -1;
        if (ahead >= 0 && ahead / P == blk) continue;
        if (blk >= num_blocks) continue;
        uint16_t* rk = ring + blk * 2 * P * 128 + (t % P) * 128;
        uint16_t* rs = rk + P * 128;
        memcpy(rk, key + i * key_stride, 256);
        memcpy(rs, score + i * score_stride, 256);
    }
}

/* ------------------------------------------------------------------------ */
/* Pool-128 online state ([C128] decode and prefill kernels)                */
/* ------------------------------------------------------------------------ */

/* State row (fp32, 384 values): max[128] | sum[128] | kv[128], where for the
 * tokens folded so far into the open 128-chunk, per channel,
 *   max = max_i s_i,  sum = sum_i e^{s_i - max},  kv = sum_i e^{s_i-max} k_i / sum.
 * Input row (fp32, 256 values): kv[128] | score[128].  Bias ape: [128][128]. */

/* Merge two partial states (m1,s1,k1) and (m2,s2,k2) of disjoint token sets,
 * as the prefill kernel merges the loaded state with the segment:
 *   M = max(m1,m2); S = s1 e^{m1-M} + s2 e^{m2-M};
 *   K = (k1 s1 e^{m1-M} + k2 s2 e^{m2-M}) / S.   Evaluated in double. */
static void merge_state(double m1, double s1, double k1, double m2, double s2, double k2,
                        double* M, double* S, double* K) {
    double mm = m1 > m2 ? m1 : m2;
    double a1 = s1 * exp(m1 - mm), a2 = s2 * exp(m2 - mm);
    *M = mm;
    *S = a1 + a2;
    *K = (k1 * a1 + k2 * a2) / (a1 + a2);
}

/* Decode: request b appends one token at global position seq_lens[b]-1, chunk
 * position c = (seq_lens[b]-1) % 128, gated score s = score + ape[c].
 *   c == 0  : state := (s, 1, k)            (first token of a chunk)
 *   c != 0  : state := merge(state, (s, 1, k))
 *   c == 127: the chunk closes: out[b] = kv (the state row is not written)
 *   else    : the state row indices[b] is written back.
 * Rows with seq_lens[b] <= 0 or indices[b] outside [0, num_slots) are
 * skipped (no read, no write). */
void orc_c128_decode(float* state, int64_t num_slots, const float* in, float* out,
                     const float* ape, const int32_t* indices, const int32_t* seq_lens,
                     int64_t batch) {
    for (int64_t b = 0; b < batch; ++b) {
        int32_t L = seq_lens[b], idx = indices[b];
        if (L <= 0 || idx < 0 || idx >= num_slots) continue;
        int c = (L - 1) % 128;
        float* st = state + (int64_t)idx * 384;
        const float* row = in + b * 256;
        float newm[128], news[128], newk[128];
        for (int d = 0; d < 128; ++d) {
            float s = row[128 + d] + ape[c * 128 + d];
            double k = row[d];
            if (c == 0) {
                newm[d] = s; news[d] = 1.0f; newk[d] = (float)k;
            } else {
                double M, S, K;
                merge_state(st[d], st[128 + d], st[256 + d], s, 1.0, k, &M, &S, &K);
                newm[d] = (float)M; news[d] = (float)S; newk[d] = (float)K;
            }
        }
        if (c == 127) {
            memcpy(out + b * 128, newk, sizeof newk);
        } else {
            memcpy(st, newm, sizeof newm);
            memcpy(st + 128, news, sizeof news);
            memcpy(st + 256, newk, sizeof newk);
        }
    }
}

/* Plan entry, 16 bytes: ragged row and global position of the segment's LAST
 * token, batch index, and the number of tokens in the segment (1..128)
 * ([C128] OnlinePrefillPlan).  All-ones marks an unused (padding) entry. */
typedef struct { uint32_t ragged_id, batch_id, position, window_len; } orc_plan;

/* Planner ([C128] plan_online_prefill_host): request b extends its sequence
 * from prefix = seq_lens[b]-extend_lens[b] to seq_lens[b]; its extend tokens
 * are rows counter..counter+extend-1 of the ragged input.  The range is cut
 * at multiples of 128.  A piece that reaches the end of its chunk is a
 * compress plan; the trailing piece that does not is the batch's single
 * write plan.  With pad, both lists are filled with all-ones entries up to
 * num_tokens.  Returns 0, or -1 when extend is not in (0, seq_len], a list
 * would exceed num_tokens, or the extends do not sum to num_tokens. */
int orc_c128_plan(const int64_t* seq_lens, const int64_t* extend_lens, int64_t batch,
                  int64_t num_tokens, orc_plan* cplan, orc_plan* wplan, int pad,
                  uint32_t* n_c, uint32_t* n_w) {
    int64_t counter = 0, nc = 0, nw = 0;
    for (int64_t b = 0; b < batch; ++b) {
        int64_t L = seq_lens[b], E = extend_lens[b];
        if (!(E > 0 && E <= L)) return -1;
        int64_t prefix = L - E;
        for (int64_t pos = prefix; pos < L;) {
            int64_t chunk_start = pos - pos % 128;
            int64_t seg_end = chunk_start + 128 < L ? chunk_start + 128 : L;
            orc_plan p;
            p.ragged_id = (uint32_t)(counter + (seg_end - 1 - prefix));
            p.batch_id = (uint32_t)b;
            p.position = (uint32_t)(seg_end - 1);
            p.window_len = (uint32_t)(seg_end - pos);
            if ((seg_end - chunk_start) == 128) {
                if (nc >= num_tokens) return -1;
                cplan[nc++] = p;
            } else {
                if (nw >= num_tokens) return -1;
                wplan[nw++] = p;
            }
            pos = seg_end;
        }
        counter += E;
    }
    if (counter != num_tokens) return -1;
    if (pad) {
        orc_plan inv = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
        for (int64_t i = nc; i < num_tokens; ++i) cplan[i] = inv;
        for (int64_t i = nw; i < num_tokens; ++i) wplan[i] = inv;
        nc = nw = num_tokens;
    }
    *n_c = (uint32_t)nc;
    *n_w = (uint32_t)nw;
    return 0;
}

/* One segment ([C128] flash_c128_online_prefill): chunk positions
 * j = off .. off+len-1 with off = position%128 + 1 - len, ragged rows
 * ragged_id-len+1 .. ragged_id.  The segment's own state is the two-pass
 * (max, sum of exp, weighted mean) over its tokens, evaluated in double; if
 * off != 0 it is merged with the state row load_indices[b].  Result in double. */
static void c128_segment(const float* state, const float* in, const float* ape,
                         const orc_plan* p, int32_t load_idx,
                         double* M, double* S, double* K) {
    uint32_t len = p->window_len;
    uint32_t off = p->position % 128u + 1u - len;
    int64_t row0 = (int64_t)p->ragged_id - (int64_t)len + 1;
    for (int d = 0; d < 128; ++d) {
        double m = -INFINITY;
        for (uint32_t i = 0; i < len; ++i) {
            float s = in[(row0 + i) * 256 + 128 + d] + ape[(off + i) * 128 + d];
            if ((double)s > m) m = s;
        }
        double den = 0.0, num = 0.0;
        for (uint32_t i = 0; i < len; ++i) {
            float s = in[(row0 + i) * 256 + 128 + d] + ape[(off + i) * 128 + d];
            double e = exp((double)s - m);
            den += e;
            num += e * (double)in[(row0 + i) * 256 + d];
        }
        double mm = m, ss = den, kk = num / den;
        if (off != 0) {
            const float* st = state + (int64_t)load_idx * 384;
            merge_state(st[d], st[128 + d], st[256 + d], mm, ss, kk, &mm, &ss, &kk);
        }
        M[d] = mm; S[d] = ss; K[d] = kk;
    }
}

/* Prefill: first every compress plan (reads state rows, writes only out rows
 * ragged_id), then every write plan (writes state rows indices[b]).  The
 * order makes every compress-plan read see the state as it was before the
 * call.  A write plan that starts mid-chunk reads row load_indices[b] as it
 * stands when that plan runs here; that is also the state before the call
 * whenever no request reads a row that another request of the call writes
 * (the device entry points require this; with load_indices NULL = indices it
 * always holds, the indices being distinct).  All-ones plans are skipped. */
void orc_c128_prefill(float* state, int64_t num_slots, const float* in, float* out,
                      const float* ape, const int32_t* indices, const int32_t* load_indices,
                      const orc_plan* cplan, uint32_t n_c, const orc_plan* wplan, uint32_t n_w) {
    (void)num_slots;
    if (!load_indices) load_indices = indices;
    double M[128], S[128], K[128];
    for (uint32_t i = 0; i < n_c; ++i) {
        const orc_plan* p = &cplan[i];
        if (p->ragged_id == 0xffffffffu) continue;
        c128_segment(state, in, ape, p, load_indices[p->batch_id], M, S, K);
        for (int d = 0; d < 128; ++d) out[(int64_t)p->ragged_id * 128 + d] = (float)K[d];
    }
    for (uint32_t i = 0; i < n_w; ++i) {
        const orc_plan* p = &wplan[i];
        if (p->ragged_id == 0xffffffffu) continue;
        c128_segment(state, in, ape, p, load_indices[p->batch_id], M, S, K);
        float* st = state + (int64_t)indices[p->batch_id] * 384;
        for (int d = 0; d < 128; ++d) {
            st[d] = (float)M[d]; st[128 + d] = (float)S[d]; st[256 + d] = (float)K[d];
        }
    }
}
