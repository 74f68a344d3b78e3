// Micro-benchmark of the gfx950 rates that set the selective scan's ALU roofline: v_exp_f32
// and fp32 FMA issue rates (16 independent chains per lane, 1-4 waves per SIMD), a scan-like
// element (1 exp + 3 FMA-class ops) to see whether exp overlaps other VALU work, plain copy /
// read bandwidth, and a check of the bf16 MFMA 16x16x32 / 32x32x16 lane layouts.
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -o /tmp/valu_rates mamba_selective_scan_02_amd/probe/valu_rates.hip && /tmp/valu_rates
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
#include <cstdlib>
#define CK(x) do{hipError_t e=(x); if(e!=hipSuccess){printf("HIP error %s at %d\n",hipGetErrorString(e),__LINE__); exit(1);}}while(0)

constexpr int CH = 16;
__global__ void exp_tp(float* out, int iters, float seed){
  float x[CH];
  for(int j=0;j<CH;j++) x[j]=seed + 0.01f*j + 1e-6f*threadIdx.x;
  for(int i=0;i<iters;i++){
#pragma unroll
    for(int j=0;j<CH;j++) x[j]=__builtin_amdgcn_exp2f(-x[j]);
  }
  float s=0; for(int j=0;j<CH;j++) s+=x[j];
  out[blockIdx.x*blockDim.x+threadIdx.x]=s;
}
__global__ void fma_tp(float* out, int iters, float seed){
  float x[CH];
  for(int j=0;j<CH;j++) x[j]=seed + 0.01f*j + 1e-6f*threadIdx.x;
  for(int i=0;i<iters;i++){
#pragma unroll
    for(int j=0;j<CH;j++) x[j]=__builtin_fmaf(x[j], 0.999f, 0.0001f);
  }
  float s=0; for(int j=0;j<CH;j++) s+=x[j];
  out[blockIdx.x*blockDim.x+threadIdx.x]=s;
}
// per iteration per chain: 1 exp + 4 dependent-ish fma/mul
__global__ void mix_tp(float* out, int iters, float seed){
  float x[CH], h[CH];
  for(int j=0;j<CH;j++){ x[j]=seed + 0.01f*j + 1e-6f*threadIdx.x; h[j]=0.f; }
  float dt = seed*0.1f, u=seed*0.3f, B=0.7f, C=0.9f, y=0.f;
  for(int i=0;i<iters;i++){
#pragma unroll
    for(int j=0;j<CH;j++){
      float a = dt * x[j];
      float dA = __builtin_amdgcn_exp2f(a);
      float dbu = u * B;
      h[j] = __builtin_fmaf(dA, h[j], dbu);
      y = __builtin_fmaf(C, h[j], y);
    }
    dt = dt*0.9999f; u = u + 1e-7f;
  }
  float s=y; for(int j=0;j<CH;j++) s+=h[j];
  out[blockIdx.x*blockDim.x+threadIdx.x]=s;
}
__global__ void copy_k(const float4* __restrict__ a, float4* __restrict__ b, size_t n){
  size_t i = blockIdx.x*(size_t)blockDim.x+threadIdx.x;
  size_t stride = (size_t)gridDim.x*blockDim.x;
  for(; i<n; i+=stride) b[i]=a[i];
}
__global__ void read_k(const float4* __restrict__ a, float* out, size_t n){
  size_t i = blockIdx.x*(size_t)blockDim.x+threadIdx.x;
  size_t stride = (size_t)gridDim.x*blockDim.x;
  float s=0;
  for(; i<n; i+=stride){ float4 v=a[i]; s+=v.x+v.y+v.z+v.w; }
  if(s==1234.5f) out[0]=s;
}
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
// A is 16x32 (m,k), B is 32x16 (k,n) given as float arrays, assumed layout:
// lane l: A[l%16][(l/16)*8 + j], B[(l/16)*8+j][l%16]; D lane l: D[(l/16)*4+j][l%16]
__global__ void mfma_layout(const float* A, const float* B, float* D){
  int l = threadIdx.x;
  bf16x8 a, b;
  for(int j=0;j<8;j++){ a[j]=(__bf16)A[(l%16)*32 + (l/16)*8+j]; b[j]=(__bf16)B[((l/16)*8+j)*16 + l%16]; }
  f32x4 c = {0,0,0,0};
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  for(int j=0;j<4;j++) D[((l/16)*4+j)*16 + l%16] = c[j];
}
// 32x32x16: A 32x16, B 16x32. assumed: lane l: A[l%32][(l/32)*8+j]; B[(l/32)*8+j][l%32];
// D: lane l holds D[ 8*(j/4) + (l/32)*4 + j%4 ][l%32], j=0..15
__global__ void mfma_layout32(const float* A, const float* B, float* D){
  int l = threadIdx.x;
  bf16x8 a, b;
  for(int j=0;j<8;j++){ a[j]=(__bf16)A[(l%32)*16 + (l/32)*8+j]; b[j]=(__bf16)B[((l/32)*8+j)*32 + l%32]; }
  f32x16 c; for(int j=0;j<16;j++) c[j]=0;
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  for(int j=0;j<16;j++) D[(8*(j/4) + (l/32)*4 + j%4)*32 + l%32] = c[j];
}

template<typename F>
float timeit(F f, int reps){
  hipEvent_t e0,e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  f(); CK(hipDeviceSynchronize());
  CK(hipEventRecord(e0));
  for(int r=0;r<reps;r++) f();
  CK(hipEventRecord(e1)); CK(hipEventSynchronize(e1));
  float ms; CK(hipEventElapsedTime(&ms,e0,e1)); return ms/reps;
}
int main(){
  hipDeviceProp_t p; CK(hipGetDeviceProperties(&p,0));
  printf("device %s arch %s CUs %d clock %d kHz mem %zu GB l2 %d lds/block %zu maxshared/cu %zu\n", p.name, p.gcnArchName, p.multiProcessorCount, p.clockRate, p.totalGlobalMem>>30, p.l2CacheSize, p.sharedMemPerBlock, p.maxSharedMemoryPerMultiProcessor);
  fflush(stdout);
  int CUs = p.multiProcessorCount;
  float* out; CK(hipMalloc(&out, sizeof(float)*CUs*16*256));
  int iters = 4096;
  for(int wpsimd : {1,2,4}){
    int blocks = CUs*4*wpsimd; // 1 wave per block
    int thr=64;
    double n = (double)blocks*thr*iters*CH;
    float t1 = timeit([&]{ exp_tp<<<blocks,thr>>>(out,iters,0.3f);},3);
    float t2 = timeit([&]{ fma_tp<<<blocks,thr>>>(out,iters,0.3f);},3);
    float t3 = timeit([&]{ mix_tp<<<blocks,thr>>>(out,iters,0.3f);},3);
    printf("waves/simd %d: exp %.3f ms -> %.3e exp/s (%.2f lanes/clk/CU @2.4GHz); fma %.3f ms -> %.3e fma/s; mix(1exp+4op) %.3f ms -> %.3e elem/s\n",
      wpsimd, t1, n/(t1*1e-3), n/(t1*1e-3)/CUs/2.4e9, t2, n/(t2*1e-3), t3, n/(t3*1e-3));
    fflush(stdout);
  }
  size_t bytes = (size_t)4<<30;
  float4 *a,*b; CK(hipMalloc(&a,bytes)); CK(hipMalloc(&b,bytes));
  CK(hipMemset(a,0,bytes)); CK(hipMemset(b,0,bytes));
  size_t n4 = bytes/16;
  for(int gm : {1,2,4,8}){
    int blocks = CUs*gm*4; int thr=256;
    float tc = timeit([&]{ copy_k<<<blocks,thr>>>(a,b,n4);},5);
    float tr = timeit([&]{ read_k<<<blocks,thr>>>(a,out,n4);},5);
    printf("grid %d: copy %.3f ms -> %.1f GB/s (r+w) ; read %.3f ms -> %.1f GB/s\n", blocks, tc, 2.0*bytes/(tc*1e-3)/1e9, tr, bytes/(tr*1e-3)/1e9);
    fflush(stdout);
  }
  // mfma layout checks
  {
    std::vector<float> A(16*32),B(32*16),D(256),R(256,0);
    for(int i=0;i<16*32;i++){ A[i]=(float)((i*7)%11-5); }
    for(int i=0;i<32*16;i++){ B[i]=(float)((i*5)%13-6); }
    for(int m=0;m<16;m++) for(int n=0;n<16;n++){ float s=0; for(int k=0;k<32;k++) s+=A[m*32+k]*B[k*16+n]; R[m*16+n]=s; }
    float *dA,*dB,*dD; CK(hipMalloc(&dA,4*512)); CK(hipMalloc(&dB,4*512)); CK(hipMalloc(&dD,4*256));
    CK(hipMemcpy(dA,A.data(),4*512,hipMemcpyHostToDevice)); CK(hipMemcpy(dB,B.data(),4*512,hipMemcpyHostToDevice));
    mfma_layout<<<1,64>>>(dA,dB,dD); CK(hipDeviceSynchronize());
    CK(hipMemcpy(D.data(),dD,4*256,hipMemcpyDeviceToHost));
    int bad=0; for(int i=0;i<256;i++) if(D[i]!=R[i]) bad++;
    printf("mfma16x16x32 layout mismatches: %d\n", bad);
  }
  {
    std::vector<float> A(32*16),B(16*32),D(1024),R(1024,0);
    for(int i=0;i<32*16;i++){ A[i]=(float)((i*7)%11-5); }
    for(int i=0;i<16*32;i++){ B[i]=(float)((i*5)%13-6); }
    for(int m=0;m<32;m++) for(int n=0;n<32;n++){ float s=0; for(int k=0;k<16;k++) s+=A[m*16+k]*B[k*32+n]; R[m*32+n]=s; }
    float *dA,*dB,*dD; CK(hipMalloc(&dA,4*512)); CK(hipMalloc(&dB,4*512)); CK(hipMalloc(&dD,4*1024));
    CK(hipMemcpy(dA,A.data(),4*512,hipMemcpyHostToDevice)); CK(hipMemcpy(dB,B.data(),4*512,hipMemcpyHostToDevice));
    mfma_layout32<<<1,64>>>(dA,dB,dD); CK(hipDeviceSynchronize());
    CK(hipMemcpy(D.data(),dD,4*1024,hipMemcpyDeviceToHost));
    int bad=0; for(int i=0;i<1024;i++) if(D[i]!=R[i]) bad++;
    printf("mfma32x32x16 layout mismatches: %d\n", bad);
  }
  printf("done\n");
  return 0;
}
