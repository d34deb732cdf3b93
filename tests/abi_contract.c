/* The boundary's prototypes as the scope table of this library states them,
 * declared again after include/aaren.h. C allows a function to be declared
 * twice only with compatible types, so this file compiles (gcc -std=c99
 * -pedantic -Werror) exactly when the header's entry points take those
 * arguments in that order. Compiled, never run. */
#include "aaren.h"

size_t aaren_scan_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d);
aaren_status aaren_scan(const void* q /*[H,d]*/, const void* k /*[B,H,N,d]*/, const void* v /*[B,H,N,d]*/,
                        void* o /*[B,H,N,d]*/, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                        aaren_dtype in_dtype, aaren_dtype out_dtype,
                        void* workspace, size_t workspace_bytes, void* hip_stream);
size_t aaren_scan_segmented_workspace_size(int64_t num_seqs, int64_t total_tokens, int64_t H, int64_t d);
aaren_status aaren_scan_segmented(const void* q /*[H,d]*/, const void* k /*[T,H,d]*/, const void* v /*[T,H,d]*/,
                        void* o /*[T,H,d]*/, const int64_t* offsets /*device, [num_seqs+1]*/,
                        int64_t num_seqs, int64_t total_tokens, int64_t H, int64_t d, float scale,
                        aaren_dtype in_dtype, aaren_dtype out_dtype,
                        void* workspace, size_t workspace_bytes, void* hip_stream);
aaren_status aaren_step(const void* q /*[H,d]*/, const void* k_t /*[S,H,d]*/, const void* v_t /*[S,H,d]*/,
                        float* m /*[S,H] in/out*/, float* u /*[S,H] in/out*/, float* w /*[S,H,d] in/out*/,
                        void* o_t /*[S,H,d] or NULL*/, int64_t S, int64_t H, int64_t d, float scale,
                        aaren_dtype in_dtype, aaren_dtype out_dtype, void* hip_stream);
aaren_status aaren_state_init(float* m, float* u, float* w, int64_t S, int64_t H, int64_t d, void* hip_stream);
size_t aaren_reduce_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d);
aaren_status aaren_reduce(const void* q /*[H,d]*/, const void* k /*[B,H,N,d]*/, const void* v /*[B,H,N,d]*/,
                        void* o /*[B,H,d]*/, float* m_out /*[B,H] or NULL*/, float* u_out /*[B,H] or NULL*/,
                        int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                        aaren_dtype in_dtype, aaren_dtype out_dtype,
                        void* workspace, size_t workspace_bytes, void* hip_stream);
const char* aaren_status_string(aaren_status s);
const char* aaren_last_error(void);
int aaren_version(void);

/* the status and dtype values */
typedef char status_values_match[(AAREN_OK == 0 && AAREN_ERR_INVALID_ARG == 1 &&
                                  AAREN_ERR_UNSUPPORTED == 2 && AAREN_ERR_ALIGNMENT == 3 &&
                                  AAREN_ERR_WORKSPACE == 4 && AAREN_ERR_HIP == 5) ? 1 : -1];
typedef char dtype_values_match[(AAREN_F32 == 0 && AAREN_BF16 == 1) ? 1 : -1];
