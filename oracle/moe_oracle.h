/*
 * moe_oracle.h -- interface of the CPU oracle (test infrastructure only).
 * Not included by, and not including, anything of the HIP library.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#define OR_MAX_EXPERTS 512
#define OR_MAX_THREADS 256

enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3 = 2 };
enum { OR_SOFTMAX = 0, OR_SIGMOID = 1 };

/* One layer as the oracle sees it.  Per-expert weight pointers let a caller
 * hand over only the experts that the listed tokens use (the others NULL). */
typedef struct {
    int64_t T, E, K, H, I;
    int scoring;                  /* OR_SOFTMAX or OR_SIGMOID */
    int renormalize;
    int n_group, topk_group;      /* n_group <= 1: ungrouped */
    double routed_scaling_factor;
    int x_dtype;                  /* OR_F32 or OR_BF16 */
    int w_dtype;                  /* OR_F32, OR_BF16 or OR_E4M3 */
    int act_fp8;                  /* quantise x and act per group of 128 */
    const void *hidden;           /* [T, H] */
    const float *logits;          /* [T, E] */
    const float *bias;            /* [E] or NULL */
    const void *const *w13;       /* E pointers to [2I, H] */
    const float *const *w13_scale;/* E pointers to [2I/128, H/128] or NULL */
    const void *const *w2;        /* E pointers to [H, I] */
    const float *const *w2_scale; /* E pointers to [H/128, I/128] or NULL */
    const void *shared_w13;       /* [2Is, H] or NULL */
    const float *shared_w13_scale;
    const void *shared_w2;        /* [H, Is] or NULL */
    const float *shared_w2_scale;
    /* activation variants (defaults: gated = 1, act_alpha = 1, clamp_limit =
     * 0, weight_on_input = 0 give the plain SiLU-and-mul layer) */
    int gated;                    /* 1: w13 is [2I, H] gate;up; 0: [I, H]     */
    double act_alpha;             /* silu_a(z) = z * sigmoid(act_alpha * z)   */
    double clamp_limit;           /* > 0: gate <= L and |up| <= L (gated)     */
    int weight_on_input;          /* 1: sum_k MLP(w_k x) instead of w_k MLP(x) */
    int64_t shared_I;             /* Is, intermediate size of the shared      */
                                  /* expert; 0 means I                        */
} or_layer;

double or_bf16_to_f64(uint16_t v);
double or_e4m3_to_f64(uint8_t v);
uint8_t or_e4m3_from_f32(float x);
void or_quant_fp8_groups(int64_t rows, int64_t cols, int64_t group,
                         const float *x, uint8_t *q, float *s);
int or_route(int64_t T, int E, int K, const float *logits, const float *bias,
             int scoring, int renorm, int G, int TG, double rsf,
             int32_t *ids, double *weights);
int or_permute(int64_t N, int E, const int32_t *ids, int32_t *offsets,
               int32_t *sorted_slots, int32_t *slot_to_row);
void or_router_logits(int64_t T, int64_t E, int64_t H, const void *hidden,
                      int x_dtype, const void *gate, int g_dtype, double *out);
int or_moe_forward_tokens(const or_layer *L, int64_t ntok,
                          const int64_t *tokens, double *out, int nthreads);

#endif
