"""What a measurement record needs to say about the GPU it ran on.

``device_facts`` reports the architecture name, compute-unit count and
memory of a torch device. ``ClockSampler`` samples the engine (sclk) and
memory (mclk) clocks, board power and temperature from the amdgpu driver's
sysfs files while a timed region runs, so that a throughput can be read
against the clock the chip actually held. Missing or unreadable files give
``None`` fields with the reason; nothing here changes a clock or a setting.
"""

from __future__ import annotations

import glob
import os
import statistics
import threading
import time


def device_facts(dev) -> dict:
    import torch

    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "gcnArchName": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "total_memory_bytes": int(p.total_memory), "pci": _pci_name(p)}


def _pci_name(p):
    try:
        return f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
    except AttributeError:
        return None


def _card_dir(pci):
    """The sysfs device directory of the GPU at PCI address `pci` (or the only amdgpu card with clock files)."""
    cands = sorted(set(os.path.realpath(os.path.dirname(f)) for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")))
    if pci:
        for c in cands:
            if os.path.basename(c).lower() == pci.lower():
                return c
    return cands[0] if len(cands) == 1 else None


def _read(path):
    try:
        with open(path) as f:
            return f.read()
    except OSError:
        return None


def _dpm_mhz(text):
    """Current level of a pp_dpm_* file: the line marked with '*', in MHz."""
    if not text:
        return None
    for ln in text.splitlines():
        if ln.strip().endswith("*"):
            num = "".join(ch for ch in ln.split(":", 1)[-1] if ch.isdigit() or ch == ".")
            try:
                return float(num)
            except ValueError:
                return None
    return None


class ClockSampler:
    """Context manager: samples sclk / mclk (MHz), power (W) and edge/junction temperature (C) every
    `period_s` seconds on a background thread; ``summary()`` gives min / median / max of each."""

    def __init__(self, dev, period_s: float = 0.005):
        self.period = period_s
        self.card = _card_dir(_pci_name(__import__("torch").cuda.get_device_properties(dev)))
        self.samples = {"sclk_mhz": [], "mclk_mhz": [], "power_w": [], "temp_c": []}
        self._stop = threading.Event()
        self._t = None
        self._files = {}
        if self.card:
            hw = sorted(glob.glob(os.path.join(self.card, "hwmon", "hwmon*")))
            h = hw[0] if hw else None
            self._files = {
                "sclk_mhz": os.path.join(self.card, "pp_dpm_sclk"),
                "mclk_mhz": os.path.join(self.card, "pp_dpm_mclk"),
                "power_w": next((p for p in (os.path.join(h, "power1_input"), os.path.join(h, "power1_average"))
                                 if h and os.path.exists(p)), None),
                "temp_c": next((p for p in sorted(glob.glob(os.path.join(h, "temp*_input"))) if h), None) if h else None,
            }

    def _sample(self):
        for key, path in self._files.items():
            if not path:
                continue
            txt = _read(path)
            if txt is None:
                continue
            if key in ("sclk_mhz", "mclk_mhz"):
                v = _dpm_mhz(txt)
            else:
                try:
                    v = float(txt.strip()) / (1e6 if key == "power_w" else 1e3)
                except ValueError:
                    v = None
            if v is not None:
                self.samples[key].append(v)

    def _run(self):
        while not self._stop.is_set():
            self._sample()
            time.sleep(self.period)

    def __enter__(self):
        if self.card:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._t:
            self._t.join()
        return False

    def summary(self) -> dict:
        out = {"source": self.card and f"{self.card}/pp_dpm_sclk, pp_dpm_mclk, hwmon"}
        if not self.card:
            out["source"] = None
            out["note"] = "no readable amdgpu sysfs clock files"
        for key, vals in self.samples.items():
            out[key] = ({"min": round(min(vals), 1), "median": round(statistics.median(vals), 1),
                         "max": round(max(vals), 1), "n": len(vals)} if vals else None)
        return out
