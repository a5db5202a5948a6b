/*
 * oq_oracle.h -- declarations of the fp64 CPU oracle (test infrastructure
 * only; see oq_oracle.c).  Nothing in the product library includes this.
 */
#ifndef OQ_ORACLE_H
#define OQ_ORACLE_H
#include <stdint.h>

enum { OQO_F32 = 0, OQO_BF16 = 1 };

uint64_t oqo_splitmix64_next(uint64_t *state);
int oqo_block_size(int d);
void oqo_plan(int d, uint64_t seed, int32_t *perm, int8_t *sign);

int oqo_codebook_unit(int bits, double *levels, double *thresholds);
int oqo_codebook(int d, int bits, double *levels, double *thresholds);
double oqo_codebook_mse(int bits, const double *levels, const double *thresholds);
int oqo_codebook_sphere(int d, int bits, double *levels, double *thresholds);
double oqo_sphere_mass(double a, double b, int d);

void oqo_fwht(double *v, int h);
int oqo_hadamard_entry(int a, int b);
void oqo_rotate_token(const double *x, int d, const int32_t *perm, const int8_t *sign,
                      int use_signs, double *z, double *norm);

int oqo_quantize_one(double z, const double *thresholds, int L);
int64_t oqo_slot_of(int64_t i, int d);
void oqo_pack_row(const uint8_t *codes, int d, int bits, uint8_t *out);
void oqo_unpack_row(const uint8_t *packed, int d, int bits, uint8_t *codes);

int oqo_rotate_quantize(const void *x, int dtype, int64_t rows, int d, uint64_t seed,
                        int use_signs, int bits, uint8_t *codes, double *norms, double *z);
int oqo_rotate_quantize_ex(const void *x, int dtype, int64_t rows, int d, uint64_t seed,
                           int use_signs, int bits, int family, uint8_t *codes, double *norms,
                           double *z);
int oqo_linear_ex(const uint8_t *a_codes, const double *a_norms, int ba,
                  const uint8_t *w_codes, const double *w_norms, int bw, int family,
                  int64_t N, int K, const int64_t *rows, int64_t nrows, double *y);
int oqo_linear(const uint8_t *a_codes, const double *a_norms, int ba,
               const uint8_t *w_codes, const double *w_norms, int bw,
               int64_t N, int K, const int64_t *rows, int64_t nrows, double *y);
int oqo_fake_quantize(const void *x, int dtype, int64_t rows, int d, uint64_t seed,
                      int use_signs, int bits, double *out, double *norms);
int oqo_rtn4_quantize(const void *W, int dtype, int64_t rows, int d, int8_t *q, float *scales);
int oqo_rtn4_linear(const void *x, int dtype, int64_t M, const int8_t *q, const float *scales,
                    int64_t N, int K, double *y);
int oqo_num_threads(void);
void oqo_set_threads(int n);
#endif
