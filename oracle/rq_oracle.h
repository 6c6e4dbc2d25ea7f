/*
 * rq_oracle.h -- plain, slow CPU reference for the ResidualQuant KV-cache codec
 * and decode attention.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the CPU-baseline leg of the benchmark may call it; the library never does.
 *
 * Everything is computed in IEEE double precision with no blocking, fusion or
 * reordering beyond what the definitions state.  It shares no code, header,
 * table or constant with the GPU library.
 *
 * Sources (web pages about "ResidualQuant: KV Cache Quantization for Looped
 * Transformers with 2-Bit Residuals"):
 *   [abstract]   arXiv abstract as listed by paperdot, single paragraph.
 *   [ai4s p1..6] ai4snews summary "ResidualQuant anchors on the final-loop KV
 *                and stores 2-bit residuals, ...", paragraphs 1..6.
 *   [agihunt]    agihunt page "KAIST's ResidualQuant: 2-bit Residual
 *                Quantization Cuts Looped Transformer KV Cache by 80%",
 *                list "Confirmed", bullets 2-3.
 *
 * Logical (unpacked) slice arrays used throughout, for ONE (K or V, batch row,
 * layer, kv head) slice with L loops and N tokens, head_dim d, group size g,
 * ng = d / g:
 *   x      uint16 [L][N][d]   BF16 bit patterns of the unquantized states
 *   codes  uint8  [L][N][d]   one code per byte (0..2^bits-1)
 *   s8,z8  uint8  [L][N][ng]  FP8 e4m3fn scale / offset bit patterns
 *   alpha  uint16 [L][N]      BF16 residual scale (0 where a loop has none)
 */
#ifndef RQ_ORACLE_H
#define RQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { RQO_MODE_RESIDUAL = 0, RQO_MODE_DIRECT = 1, RQO_MODE_CHAINED = 2 };
enum { RQO_ALPHA_LS = 0, RQO_ALPHA_NORM_RATIO = 1, RQO_ALPHA_ONE = 2 };

typedef struct {
  int d;              /* head_dim */
  int g;              /* quantization group size along head_dim */
  int P;              /* loops per group; the anchor is the last loop of a group */
  int anchor_bits;    /* bits of the anchor (or, in direct mode, of the anchor-position loop) */
  int residual_bits;  /* bits of every other loop */
  int mode;           /* RQO_MODE_RESIDUAL, RQO_MODE_DIRECT or RQO_MODE_CHAINED */
  int alpha_mode;     /* RQO_ALPHA_* (residual and chained modes) */
  int rotate;         /* 1: rotate residuals with H; 0: identity */
} rqo_params;

/* ---- number formats ---- */
double   rqo_fp8_decode(uint8_t code);
uint8_t  rqo_fp8_encode(double x);
double   rqo_bf16_decode(uint16_t code);
uint16_t rqo_bf16_encode(double x);

/* element-wise array forms of the four conversions above */
void rqo_fp8_decode_n(const uint8_t* in, long n, double* out);
void rqo_fp8_encode_n(const double* in, long n, uint8_t* out);
void rqo_bf16_decode_n(const uint16_t* in, long n, double* out);
void rqo_bf16_encode_n(const double* in, long n, uint16_t* out);

/* ---- rotation H = B * diag(signs) ----
 * B is block diagonal over the binary decomposition of d (largest block first),
 * each block the n x n Sylvester Walsh-Hadamard matrix times 1/sqrt(n).
 * rqo_rotation_matrix writes H row-major (d*d); rqo_rotate computes y = H r and
 * rqo_rotate_t computes r = H^T y as the exact +-1 sums followed by the scale.
 * Functions below that take `signs` ignore it when residuals are not rotated. */
int rqo_rotation_matrix(int d, const int8_t* signs, double* H);
int rqo_rotate(int d, const int8_t* signs, const double* r, double* y);
int rqo_rotate_t(int d, const int8_t* signs, const double* y, double* r);

/* ---- group quantizer and its inverse ---- */
void rqo_quant_group(const double* x, int g, int bits,
                     uint8_t* s8, uint8_t* z8, uint8_t* codes);
void rqo_quant_vector(const double* x, int d, int g, int bits,
                      uint8_t* codes, uint8_t* s8, uint8_t* z8);
void rqo_dequant_vector(const uint8_t* codes, const uint8_t* s8, const uint8_t* z8,
                        int d, int g, double* out);

/* ---- one loop group of one token vector ---- */
int rqo_encode_group(const rqo_params* p, const double* x /* [P][d] */,
                     const int8_t* signs /* [d] */,
                     uint8_t* codes /* [P][d] */, uint8_t* s8 /* [P][ng] */,
                     uint8_t* z8 /* [P][ng] */, uint16_t* alpha /* [P] */);
int rqo_reconstruct_group(const rqo_params* p, const uint8_t* codes,
                          const uint8_t* s8, const uint8_t* z8,
                          const uint16_t* alpha, const int8_t* signs, int j,
                          double* out /* [d] */);

/* ---- whole slices (see header comment for array layouts) ---- */
int rqo_encode_slice(const rqo_params* p, int L, int N, const uint16_t* x,
                     const int8_t* signs, uint8_t* codes, uint8_t* s8, uint8_t* z8,
                     uint16_t* alpha);
int rqo_reconstruct_slice(const rqo_params* p, int L, int N,
                          const uint8_t* codes, const uint8_t* s8, const uint8_t* z8,
                          const uint16_t* alpha, const int8_t* signs, int loop,
                          int t0, int t1, double* out /* [t1-t0][d] */);

/* ---- attention of one query over tokens [0, n) ---- */
int rqo_attention_dense(int n, int d, const double* q, const double* Khat,
                        const double* Vhat, double scale, double* out);
int rqo_attention_slice(const rqo_params* p, int L, int N, int n, int loop,
                        const uint16_t* q_bf16, const int8_t* signs_k,
                        const int8_t* signs_v,
                        const uint8_t* kc, const uint8_t* ks, const uint8_t* kz,
                        const uint16_t* ka,
                        const uint8_t* vc, const uint8_t* vs, const uint8_t* vz,
                        const uint16_t* va,
                        double scale, int fused, double* out /* [d] */);

/* ---- storage accounting ---- */
double rqo_bits_per_element(int anchor_bits, int residual_bits, int g, int d, int P,
                            int with_alpha);

#ifdef __cplusplus
}
#endif
#endif
