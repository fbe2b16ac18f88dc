/* Host fills of the seeded generator (see qsagen_core.h). */
#include <stddef.h>
#include <stdint.h>
#include "qsagen_core.h"

void qsagen_host_normal_f32(float *dst, uint64_t n, uint64_t stream, uint64_t e0)
{
    long long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < (long long)n; ++i)
        dst[i] = qsagen_normal(stream, e0 + (uint64_t)i);
}

void qsagen_host_unit_f32(float *dst, uint64_t n, uint64_t stream, uint64_t e0, float offset)
{
    long long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < (long long)n; ++i)
        dst[i] = offset + qsagen_unit(stream, e0 + (uint64_t)i);
}

/* Gather rows: dst[r][j] = normal(stream, rows[r] * row_len + j). */
void qsagen_host_normal_rows_f32(float *dst, const int64_t *rows, uint64_t n_rows,
                                 uint64_t row_len, uint64_t stream)
{
    long long r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < (long long)n_rows; ++r)
        for (uint64_t j = 0; j < row_len; ++j)
            dst[(uint64_t)r * row_len + j] =
                qsagen_normal(stream, (uint64_t)rows[r] * row_len + j);
}

uint64_t qsagen_host_stream(uint64_t seed, uint64_t tensor_id)
{
    return qsagen_stream(seed, tensor_id);
}

uint64_t qsagen_host_mix(uint64_t x)
{
    return qsagen_mix(x);
}
